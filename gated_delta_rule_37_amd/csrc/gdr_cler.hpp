// gdr_cler.hpp -- per-piece arithmetic of the error-routing epilogue (CLER-H).
//
// CLER-H (popular article on the study, cross-layer section) adds the write
// error of the delta rule, e_t = v_t - (Diag(alpha_t) S_{t-1})^T k_t, into the
// hidden stream: h[t, h*dv + j] += lam[h*dv + j] * e_t[j].  The chunked form
// keeps u_t = beta_t e_t (the rows of U), so e_t = u_t / beta_t; beta == 0 is
// outside the domain.
//
// The saved U is in fragment order: piece p (eight consecutive columns of one
// row) is lane p % 64 of fragment p / 64 = (row tile, 32-column step).  The
// kernels below walk the pieces of a chunk, which keeps the U reads contiguous
// and lets 256 threads cover whole 128-byte lines of the hidden rows.
#pragma once

#include "gdr_common.hpp"
#include "gdr_launch.hpp"

#include <type_traits>

namespace gdr {

template <int D>
__device__ __forceinline__ void frag_piece(int p, int& pos, int& j) {
    const int f = p >> 6, l = p & 63;
    pos = 16 * (f / (D / 32)) + (l & 15);
    j = 32 * (f % (D / 32)) + 8 * (l >> 4);
}

// h[0..7] += lam[0..7] * u[0..7] / beta for one piece of a hidden row.
template <typename InT>
__device__ __forceinline__ void cler_add8(InT* hrow, const float (&u)[8], const float (&lm)[8], float beta) {
    float hv[8];
    load8f(hrow, hv);
    const float ib = 1.f / beta;
#pragma unroll
    for (int e = 0; e < 8; ++e) hv[e] = __builtin_fmaf(lm[e], u[e] * ib, hv[e]);
    store8f(hrow, hv);
}

template <int D, bool IN_F32>
struct ClerLayout {
    using OpT = typename std::conditional<IN_F32, float, _Float16>::type;
    static constexpr int PAD = 16 / sizeof(OpT);
    static constexpr int LDE = D + PAD;       // dE [64][D] row stride
    static constexpr int LDT = CHUNK + PAD;   // [x][64] row stride (M^T, dE^T)
    // the post-gradient terms: dE [64][LDE], then one [32] column-sum row per wave
    static constexpr int COLRED = CHUNK * LDE * (int)sizeof(OpT);
    static constexpr int POST_BYTES = COLRED + 8 * 32 * 4;  // up to eight waves
};

// The first half of the write errors' terms between the two gradient stages
// (NT threads of the chunk's workgroup): dE = lam * dh into LDS (smem, [64][LDE]
// in operand precision, rows past the end zero) and the scale gradient's
// partial row of this chunk, sum_t dh_t e_t with e = U / beta (if partial is not
// NULL).  Ends with a barrier: dE is visible to every wave.
template <int D, bool IN_F32, int NT>
__device__ __forceinline__ void cler_build_dE(int64_t T, int H, int64_t NC, const ChunkWs& ws,
                                              const float* __restrict__ beta, const float* __restrict__ lam,
                                              const void* __restrict__ dh_, float* __restrict__ partial,
                                              ChunkRange cr, char* smem) {
    using Lc = ClerLayout<D, IN_F32>;
    using OpT = typename Lc::OpT;
    using InT = typename InType<IN_F32>::T;
    constexpr int LDE = Lc::LDE, KQ = D / 32, NW = NT / 64, NPT = CHUNK * D / 8 / NT;
    static_assert(NT % 256 == 0 && NW % KQ == 0 && CHUNK * D / 8 % NT == 0, "thread count");
    static_assert(NW <= 8, "the column-sum table holds eight waves");
    OpT* sE = reinterpret_cast<OpT*>(smem);
    float (*colred)[32] = reinterpret_cast<float (*)[32]>(smem + Lc::COLRED);

    int64_t bh, c;
    range_block(cr, bh, c);
    const int64_t ch = bh * NC + c;
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh % H);
    const int tid = threadIdx.x, wid = tid >> 6, l16 = tid & 15;
    const int64_t nvalid64 = T - c * CHUNK;
    const int nvalid = nvalid64 < CHUNK ? static_cast<int>(nvalid64) : CHUNK;
    const OpT* U = reinterpret_cast<const OpT*>(ws.Usave) + ch * CHUNK * D;
    const InT* dh = reinterpret_cast<const InT*>(dh_);

    // pieces of U (fragment order) with the matching dh: dE rows into LDS and
    // the per-column sums of dh . e.  A thread's columns are the same in every
    // piece it takes (the fragment index advances by NW, a multiple of the
    // 32-column steps per row).
    float col[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) col[e] = 0.f;
    int jcol = 0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const int p = i * NT + tid;
        int pos, j;
        frag_piece<D>(p, pos, j);
        jcol = j;
        float g[8], lm[8], u[8];
        load_lam8(lam, static_cast<int64_t>(h) * D + j, lm);
        if (pos < nvalid) {
            const int64_t t = c * CHUNK + pos;
            load8f(dh + ((b * T + t) * H + h) * D + j, g);
            load8f(U + p * 8, u);
            const float ib = 1.f / beta[(b * T + t) * H + h];
#pragma unroll
            for (int e = 0; e < 8; ++e) col[e] = __builtin_fmaf(g[e], u[e] * ib, col[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) g[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) sE[pos * LDE + j + e] = static_cast<OpT>(lm[e] * g[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        col[e] += __shfl_xor(col[e], 1);
        col[e] += __shfl_xor(col[e], 2);
        col[e] += __shfl_xor(col[e], 4);
        col[e] += __shfl_xor(col[e], 8);
    }
    if (l16 == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) colred[wid][(jcol & 31) + e] = col[e];
    }
    __syncthreads();
    if (partial && tid < D) {
        // column tid lies in 32-column step tid / 32, held by the waves w with w % KQ == step
        const int step = tid >> 5;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            if (w % KQ == step) s += colred[w][tid & 31];
        partial[(b * NC + c) * (static_cast<int64_t>(H) * D) + static_cast<int64_t>(h) * D + tid] = s;
    }
}

// Between the two gradient stages of a chunk (NT threads of its workgroup, on
// an LDS buffer of ClerLayout::POST_BYTES), with the first stage's dKt and dP
// in the workspace: the write errors' own terms, e = (V - Kt S) - M U:
//   dKt -= dE S^T,   dP -= strict_tril(dE U^T),
// and the scale gradient's partial row of this chunk (cler_build_dE).
template <int D, bool IN_F32, int NT>
__device__ __forceinline__ void cler_post_body(int64_t T, int H, int64_t NC, const ChunkWs& ws,
                                               const float* __restrict__ beta, const float* __restrict__ lam,
                                               const void* __restrict__ dh_, float* __restrict__ partial,
                                               ChunkRange cr, char* smem) {
    using Lc = ClerLayout<D, IN_F32>;
    using OpT = typename Lc::OpT;
    constexpr int LDE = Lc::LDE, KQ = D / 32, NW = NT / 64;
    const OpT* sE = reinterpret_cast<const OpT*>(smem);

    int64_t bh, c;
    range_block(cr, bh, c);
    const int64_t ch = bh * NC + c;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const OpT* U = reinterpret_cast<const OpT*>(ws.Usave) + ch * CHUNK * D;
    const OpT* Ss = reinterpret_cast<const OpT*>(ws.Ssnap) + ch * D * D;
    OpT* gKt = static_cast<OpT*>(ws.gKt) + ch * CHUNK * D;
    // this wave's state-row tile of dKt (see below): its sixteen dKt values and
    // its S fragments are loaded first, so that they arrive while dE is built
    static_assert(D / 16 == NW, "one state-row tile of dKt per wave");
    const int dt = wid;
    OpT cur[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) cur[rt][e] = gKt[(16 * rt + 4 * g4 + e) * D + 16 * dt + l16];
    Frag<OpT> fs[KQ];
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) fs[kq].load(Ss + ((dt * KQ + kq) * 64 + lane) * 8);

    cler_build_dE<D, IN_F32, NT>(T, H, NC, ws, beta, lam, dh_, partial, cr, smem);

    // dKt -= dE S^T: wave w takes the state-row tile dt = w for all four position
    // tiles (S fragments read once).  Its dKt values were loaded at the start and
    // are stored after all four products, so the read-modify-writes do not wait
    // on one another.
    {
        float4v acc[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            acc[rt] = zero4();
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq) {
                Frag<OpT> fe;
                fe.load(sE + (16 * rt + l16) * LDE + 32 * kq + 8 * g4);
                mma(fe, fs[kq], acc[rt]);
            }
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                gKt[(16 * rt + 4 * g4 + e) * D + 16 * dt + l16] = from_f32<OpT>(to_f32(cur[rt][e]) - acc[rt][e]);
    }
    // dP -= strict_tril(dE U^T): wave w < 4 takes position-row tile w and the
    // column tiles up to it, its dP values loaded first in the same way
    if (wid < 4) {
        OpT* gP = static_cast<OpT*>(ws.gP) + ch * CHUNK * CHUNK;
        const int at = wid;
        OpT cp[4][4];
#pragma unroll
        for (int xt = 0; xt < 4; ++xt)
#pragma unroll
            for (int e = 0; e < 4; ++e) cp[xt][e] = gP[(16 * at + 4 * g4 + e) * CHUNK + 16 * xt + l16];
        float4v acc[4];
#pragma unroll
        for (int xt = 0; xt < 4; ++xt) {
            acc[xt] = zero4();
            if (xt <= at) {
#pragma unroll
                for (int kq = 0; kq < KQ; ++kq) {
                    Frag<OpT> fe, fu;
                    fe.load(sE + (16 * at + l16) * LDE + 32 * kq + 8 * g4);
                    fu.load(U + ((xt * KQ + kq) * 64 + lane) * 8);
                    mma(fe, fu, acc[xt]);
                }
            }
        }
#pragma unroll
        for (int xt = 0; xt < 4; ++xt) {
            const int x = 16 * xt + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int a = 16 * at + 4 * g4 + e;
                if (xt <= at && x < a) gP[a * CHUNK + x] = from_f32<OpT>(to_f32(cp[xt][e]) - acc[xt][e]);
            }
        }
    }
}

}  // namespace gdr
