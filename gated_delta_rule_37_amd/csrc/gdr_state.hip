// gdr_state.hip -- inter-chunk state propagation with the fused output.
//
// Chunks are chained sequentially (each chunk keeps its own start state, KDA
// blog section 6.1).  For chunk c with start state S (dk x dv, fp32):
//   U   = Ut_c - W_c S                 (beta-scaled write error of every token)
//   O   = scale (Qt_c S + A_c U)       (read-out after each token's write)
//   S  <- Diag(gamma_c) S + Kb_c^T U   (state at the chunk's end)
// Columns of S are independent in all three lines, so a head's state is split
// into dv slices of 16 columns, one workgroup per (batch, head, slice): the
// only sequential work left is one small product chain per chunk.  The state
// stays in registers as fp32 matrix-core accumulators for the whole sequence;
// a transposed fp16 (or fp32) copy in LDS feeds the next chunk's products.  The
// next chunk's operand fragments are prefetched into registers while the
// current chunk computes (double buffering, KDA blog section 6.2).
//
// Workgroups of one head are placed on one XCD (workgroups are dealt to the
// eight XCDs round robin), so the chunk operands shared by a head's slices are
// fetched into that XCD's L2 once.
#include "gdr_common.hpp"
#include "gdr_launch.hpp"

#include <type_traits>

namespace gdr {

template <int D, bool IN_F32>
struct StateCfg {
    using OpT = typename std::conditional<IN_F32, float, _Float16>::type;
    static constexpr int NS = 16;         // columns per slice
    static constexpr int NSL = D / NS;    // slices per head
    static constexpr int PAD = 16 / sizeof(OpT);
    static constexpr int LDS_S = D + PAD;      // row stride of the transposed state slice [NS][D]
    static constexpr int LDS_U = CHUNK + PAD;  // row stride of the transposed U slice [NS][64]
    static constexpr int SRT = D / 64;         // 16-row state tiles per wave
};

template <int D, bool IN_F32>
struct ChunkFrags {
    using OpT = typename StateCfg<D, IN_F32>::OpT;
    static constexpr int SRT = StateCfg<D, IN_F32>::SRT;
    Frag<OpT> w[D / 32], q[D / 32], a[2], kb[SRT][2];
    float ut[4];
    float gam[SRT][4];
};

template <int D, bool IN_F32>
__device__ __forceinline__ void load_chunk(ChunkFrags<D, IN_F32>& f, const ChunkWs& ws, int64_t ch,
                                           int j0, int wid, int l16, int g4) {
    using Cfg = StateCfg<D, IN_F32>;
    using OpT = typename Cfg::OpT;
    const OpT* W = reinterpret_cast<const OpT*>(ws.W) + ch * CHUNK * D + (16 * wid + l16) * D + 8 * g4;
    const OpT* Q = reinterpret_cast<const OpT*>(ws.Qt) + ch * CHUNK * D + (16 * wid + l16) * D + 8 * g4;
#pragma unroll
    for (int kq = 0; kq < D / 32; ++kq) {
        f.w[kq].load(W + 32 * kq);
        f.q[kq].load(Q + 32 * kq);
    }
    const OpT* A = reinterpret_cast<const OpT*>(ws.A) + ch * CHUNK * CHUNK + (16 * wid + l16) * CHUNK + 8 * g4;
    f.a[0].load(A);
    if (wid >= 2) f.a[1].load(A + 32);
    else f.a[1].zero();
    const OpT* KbT = reinterpret_cast<const OpT*>(ws.KbT) + ch * D * CHUNK;
#pragma unroll
    for (int m = 0; m < Cfg::SRT; ++m) {
        const OpT* row = KbT + (wid * (D / 4) + 16 * m + l16) * CHUNK + 8 * g4;
        f.kb[m][0].load(row);
        f.kb[m][1].load(row + 32);
#pragma unroll
        for (int e = 0; e < 4; ++e) f.gam[m][e] = ws.gam[ch * D + wid * (D / 4) + 16 * m + 4 * g4 + e];
    }
    const OpT* Ut = reinterpret_cast<const OpT*>(ws.Ut) + ch * CHUNK * D + j0 + l16;
#pragma unroll
    for (int e = 0; e < 4; ++e) f.ut[e] = to_f32(Ut[(16 * wid + 4 * g4 + e) * D]);
}

template <typename OpT>
__device__ __forceinline__ void st4(OpT* dst, const float4v& v) {
    if constexpr (sizeof(OpT) == 2) {
        half4 h;
        h[0] = static_cast<_Float16>(v[0]); h[1] = static_cast<_Float16>(v[1]);
        h[2] = static_cast<_Float16>(v[2]); h[3] = static_cast<_Float16>(v[3]);
        *reinterpret_cast<half4*>(dst) = h;
    } else {
        *reinterpret_cast<float4v*>(dst) = v;
    }
}

template <int D, bool IN_F32, bool OUT_F32, bool SAVE>
__global__ __launch_bounds__(256) void state_fwd_kernel(int64_t T, int H, int64_t NC, float scale,
                                                        ChunkWs ws, const float* S0,
                                                        float* ST, void* __restrict__ o_) {
    // S0 and ST may alias: each workgroup reads its slice of S0 before it
    // writes the same slice of ST, and slices of different workgroups are disjoint.
    using Cfg = StateCfg<D, IN_F32>;
    using OpT = typename Cfg::OpT;
    using OutT = typename InType<OUT_F32>::T;
    constexpr int NSL = Cfg::NSL, SRT = Cfg::SRT, LDS_S = Cfg::LDS_S, LDS_U = Cfg::LDS_U;

    __shared__ __attribute__((aligned(16))) OpT s_S[Cfg::NS * LDS_S];  // S slice, [j][d]
    __shared__ __attribute__((aligned(16))) OpT s_U[Cfg::NS * LDS_U];  // U slice, [j][pos]

    const int64_t nblk = gridDim.x;
    int64_t lid = blockIdx.x;
    if (nblk % 8 == 0) lid = (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
    const int64_t bh = lid / NSL;
    const int j0 = static_cast<int>(lid % NSL) * Cfg::NS;
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh % H);

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    OutT* o = reinterpret_cast<OutT*>(o_);

    // state tile m of this wave: rows wid*D/4 + 16m + 4*g4 + e, column j0 + l16
    float4v S[SRT];
#pragma unroll
    for (int m = 0; m < SRT; ++m) {
        const int d0 = wid * (D / 4) + 16 * m + 4 * g4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[m][e] = S0 ? S0[(bh * D + d0 + e) * D + j0 + l16] : 0.f;
        st4<OpT>(s_S + l16 * LDS_S + d0, S[m]);
    }
    __syncthreads();

    ChunkFrags<D, IN_F32> cur, nxt;
    if (NC > 0) load_chunk<D, IN_F32>(cur, ws, bh * NC, j0, wid, l16, g4);

#pragma unroll 1
    for (int64_t c = 0; c < NC; ++c) {
        const int64_t ch = bh * NC + c;
        if (c + 1 < NC) load_chunk<D, IN_F32>(nxt, ws, ch + 1, j0, wid, l16, g4);

        if constexpr (SAVE) {
            // chunk-start state snapshot [D][D] in operand precision
            OpT* snap = reinterpret_cast<OpT*>(ws.Ssnap) + ch * D * D;
#pragma unroll
            for (int m = 0; m < SRT; ++m) {
                const int d0 = wid * (D / 4) + 16 * m + 4 * g4;
#pragma unroll
                for (int e = 0; e < 4; ++e) snap[(d0 + e) * D + j0 + l16] = from_f32<OpT>(S[m][e]);
            }
        }

        // U = Ut - W S and the inter-chunk part of the output, O = Qt S
        float4v u = zero4(), oacc = zero4();
#pragma unroll
        for (int kq = 0; kq < D / 32; ++kq) {
            Frag<OpT> fs;
            fs.load(s_S + l16 * LDS_S + 32 * kq + 8 * g4);
            mma(cur.w[kq], fs, u);
            mma(cur.q[kq], fs, oacc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = cur.ut[e] - u[e];
        st4<OpT>(s_U + l16 * LDS_U + 16 * wid + 4 * g4, u);
        if constexpr (SAVE) {
            OpT* us = reinterpret_cast<OpT*>(ws.Usave) + ch * CHUNK * D + j0 + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) us[(16 * wid + 4 * g4 + e) * D] = from_f32<OpT>(u[e]);
        }
        __syncthreads();

        // intra-chunk part of the output, O += A U
        {
            Frag<OpT> fu;
            fu.load(s_U + l16 * LDS_U + 8 * g4);
            mma(cur.a[0], fu, oacc);
            if (wid >= 2) {
                fu.load(s_U + l16 * LDS_U + 32 + 8 * g4);
                mma(cur.a[1], fu, oacc);
            }
            const int64_t tbase = c * CHUNK + 16 * wid + 4 * g4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t t = tbase + e;
                if (t < T) o[((b * T + t) * H + h) * D + j0 + l16] = from_f32<OutT>(scale * oacc[e]);
            }
        }

        // S <- Diag(gamma) S + Kb^T U
        {
            Frag<OpT> fu0, fu1;
            fu0.load(s_U + l16 * LDS_U + 8 * g4);
            fu1.load(s_U + l16 * LDS_U + 32 + 8 * g4);
#pragma unroll
            for (int m = 0; m < SRT; ++m) {
#pragma unroll
                for (int e = 0; e < 4; ++e) S[m][e] *= cur.gam[m][e];
                mma(cur.kb[m][0], fu0, S[m]);
                mma(cur.kb[m][1], fu1, S[m]);
                st4<OpT>(s_S + l16 * LDS_S + wid * (D / 4) + 16 * m + 4 * g4, S[m]);
            }
        }
        __syncthreads();
        cur = nxt;
    }

    if (ST) {
#pragma unroll
        for (int m = 0; m < SRT; ++m) {
            const int d0 = wid * (D / 4) + 16 * m + 4 * g4;
#pragma unroll
            for (int e = 0; e < 4; ++e) ST[(bh * D + d0 + e) * D + j0 + l16] = S[m][e];
        }
    }
}

template <int D, bool IN_F32, bool OUT_F32>
static hipError_t launch_state_t(int64_t B, int64_t T, int H, int64_t NC, float scale,
                                 const ChunkWs& ws, const float* S0, float* ST, void* o, bool save,
                                 hipStream_t stream) {
    const int64_t nblk = B * H * StateCfg<D, IN_F32>::NSL;
    if (nblk == 0) return hipSuccess;
    if (save)
        hipLaunchKernelGGL((state_fwd_kernel<D, IN_F32, OUT_F32, true>), dim3((unsigned)nblk), dim3(256), 0,
                           stream, T, H, NC, scale, ws, S0, ST, o);
    else
        hipLaunchKernelGGL((state_fwd_kernel<D, IN_F32, OUT_F32, false>), dim3((unsigned)nblk), dim3(256), 0,
                           stream, T, H, NC, scale, ws, S0, ST, o);
    return hipGetLastError();
}

hipError_t launch_state_fwd(int D, bool in_f32, bool out_f32, int64_t B, int64_t T, int H,
                            int64_t NC, float scale, const ChunkWs& ws, const float* S0,
                            float* ST, void* o, bool save_for_backward, hipStream_t stream) {
    if (D == 64) {
        if (in_f32) {
            if (out_f32) return launch_state_t<64, true, true>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, stream);
            return launch_state_t<64, true, false>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, stream);
        }
        if (out_f32) return launch_state_t<64, false, true>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, stream);
        return launch_state_t<64, false, false>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, stream);
    }
    if (in_f32) {
        if (out_f32) return launch_state_t<128, true, true>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, stream);
        return launch_state_t<128, true, false>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, stream);
    }
    if (out_f32) return launch_state_t<128, false, true>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, stream);
    return launch_state_t<128, false, false>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, stream);
}

}  // namespace gdr
