// gdr_bwd_state.hip -- reverse state pass of the chunked backward.
//
// Reverse mode of the chunk recurrence (forward, per chunk c with start state S):
//   U = Ut - W S,   O = Qt S + A U,   S' = Diag(gamma) S + Kb^T U.
// Carrying dS' = dL/dS' backwards (dO already multiplied by the output scale):
//   dU = A^T dO + Kb dS'
//   dS = Qt^T dO + Diag(gamma) dS' - W^T dU
// Columns of the state are again independent, so the pass is split into dv
// slices of 16 columns exactly like the forward pass.  Per chunk it saves the
// chunk-end gradient dS' and dU (fragment order, for the gradient kernels); the
// gradient that reaches the initial state is dS0.
//
// With the error-routing epilogue (CLER-H) the write errors
// E = (V - Kt S) - M U (M = strict_tril(P)) feed the hidden stream, and their
// gradient dE = lam * dh adds dU -= M^T dE and dS -= Kt^T dE.  The saved dU
// (read by the gradient kernels) is dU - M^T dE, with M^T dE formed before this
// pass.  The state update uses the equivalent
//   dS -= W^T (dU + dE / beta)    [W^T (dE / beta + M^T dE) = Kt^T dE]
// which needs no Kt: only dh and beta are staged besides M^T dE.
#include "gdr_common.hpp"
#include "gdr_launch.hpp"

#include <type_traits>

namespace gdr {

template <int D, bool IN_F32>
struct BwdCfg {
    using OpT = typename std::conditional<IN_F32, float, _Float16>::type;
    using InT = typename InType<IN_F32>::T;
    static constexpr int NS = 16;
    static constexpr int NSL = D / NS;
    static constexpr int PAD = 16 / sizeof(OpT);
    static constexpr int LDS_S = D + PAD;
    static constexpr int LDS_U = CHUNK + PAD;
    static constexpr int SRT = D / 64;
};

// Gradient arriving at the hidden stream of the error-routing epilogue (dh NULL:
// no epilogue) with its scale (NULL: ones) and the betas.
struct ClerBwd {
    const void* dh;
    const float* lam;
    const float* beta;
};

template <int D, bool IN_F32>
struct BwdFrags {
    using OpT = typename BwdCfg<D, IN_F32>::OpT;
    using InT = typename BwdCfg<D, IN_F32>::InT;
    static constexpr int SRT = BwdCfg<D, IN_F32>::SRT;
    Frag<OpT> at[2], kb[D / 32], qtt[SRT][2], wt[SRT][2];
    float gam[SRT][4];
    InT dO[4];
    InT dh[4];    // error-routing epilogue only
    float bt[4];
    OpT mt[4];
};

// Loads the operands of chunk c (fragment order, contiguous per fragment) and
// this lane's four dO values (rows 16*wid + 4*g4 + e, column j0 + l16).
template <int D, bool IN_F32, bool CLER>
__device__ __forceinline__ void load_bwd(BwdFrags<D, IN_F32>& f, const ChunkWs& ws, int64_t ch, int64_t c,
                                         int64_t b, int64_t T, int H, int h, const void* dO_, int j0, int wid,
                                         int lane, const ClerBwd& cl) {
    using Cfg = BwdCfg<D, IN_F32>;
    using OpT = typename Cfg::OpT;
    using InT = typename Cfg::InT;
    const OpT* AT = reinterpret_cast<const OpT*>(ws.AT) + ch * CHUNK * CHUNK;
    f.at[0].load(AT + ((wid * 2 + 0) * 64 + lane) * 8);
    f.at[1].load(AT + ((wid * 2 + 1) * 64 + lane) * 8);
    const OpT* Kb = reinterpret_cast<const OpT*>(ws.Kb) + ch * CHUNK * D;
#pragma unroll
    for (int kq = 0; kq < D / 32; ++kq) f.kb[kq].load(Kb + ((wid * (D / 32) + kq) * 64 + lane) * 8);
    const OpT* QtT = reinterpret_cast<const OpT*>(ws.QtT) + ch * D * CHUNK;
    const OpT* WT = reinterpret_cast<const OpT*>(ws.WT) + ch * D * CHUNK;
#pragma unroll
    for (int m = 0; m < Cfg::SRT; ++m) {
        const int rt = wid * (D / 64) + m;
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
            f.qtt[m][kq].load(QtT + ((rt * 2 + kq) * 64 + lane) * 8);
            f.wt[m][kq].load(WT + ((rt * 2 + kq) * 64 + lane) * 8);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) f.gam[m][e] = ws.gam[ch * D + 16 * rt + 4 * (lane >> 4) + e];
    }
    const InT* dO = reinterpret_cast<const InT*>(dO_);
    const int64_t tb = c * CHUNK + 16 * wid + 4 * (lane >> 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t t = (tb + e < T) ? tb + e : T - 1;  // clamped; zeroed at use
        f.dO[e] = dO[((b * T + t) * H + h) * D + j0 + (lane & 15)];
        if constexpr (CLER) {
            f.dh[e] = reinterpret_cast<const InT*>(cl.dh)[((b * T + t) * H + h) * D + j0 + (lane & 15)];
            f.bt[e] = cl.beta[(b * T + t) * H + h];
            f.mt[e] = reinterpret_cast<const OpT*>(ws.Mt)[(ch * CHUNK + 16 * wid + 4 * (lane >> 4) + e) * D + j0 +
                                                          (lane & 15)];
        }
    }
}

template <typename OpT>
__device__ __forceinline__ void st4b(OpT* dst, const float4v& v) {
    if constexpr (sizeof(OpT) == 2) {
        half4 hv;
        hv[0] = from_f32<_Float16>(v[0]); hv[1] = from_f32<_Float16>(v[1]);
        hv[2] = from_f32<_Float16>(v[2]); hv[3] = from_f32<_Float16>(v[3]);
        *reinterpret_cast<half4*>(dst) = hv;
    } else {
        *reinterpret_cast<float4v*>(dst) = v;
    }
}

template <typename OpT>
__device__ __forceinline__ void st8(OpT* dst, const OpT (&v)[8]) {
    if constexpr (sizeof(OpT) == 2) {
        half8 hv;
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = v[e];
        *reinterpret_cast<half8*>(dst) = hv;
    } else {
        float4v a, c;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = v[e];
            c[e] = v[4 + e];
        }
        reinterpret_cast<float4v*>(dst)[0] = a;
        reinterpret_cast<float4v*>(dst)[1] = c;
    }
}

template <int D, bool IN_F32, bool CLER>
__device__ __forceinline__ void bwd_step(const BwdFrags<D, IN_F32>& cur, int64_t c, int64_t T, int64_t bh,
                                         int64_t NC, int j0, int wid, int lane, float scale, float lamj,
                                         const ChunkWs& ws,
                                         float4v (&dS)[BwdCfg<D, IN_F32>::SRT],
                                         typename BwdCfg<D, IN_F32>::OpT* s_dS,
                                         typename BwdCfg<D, IN_F32>::OpT* s_dO,
                                         typename BwdCfg<D, IN_F32>::OpT* s_dU,
                                         typename BwdCfg<D, IN_F32>::OpT* s_dUE) {
    using Cfg = BwdCfg<D, IN_F32>;
    using OpT = typename Cfg::OpT;
    constexpr int SRT = Cfg::SRT, LDS_S = Cfg::LDS_S, LDS_U = Cfg::LDS_U;
    const int l16 = lane & 15, g4 = lane >> 4, tid = wid * WAVE + lane;
    const int64_t ch = bh * NC + c;

    // chunk-end gradient dS' of this chunk, fragment order (rows d, k = column):
    // each 16-lane group 16 rows and 8 of the columns
    if (tid < 2 * D) {
        const int grp = tid >> 4, d0 = 16 * (grp % (D / 16)), hf = grp / (D / 16);
        OpT vals[8];
        lds_column8<LDS_S>(s_dS, 8 * hf, d0, lane, vals);
        st8(reinterpret_cast<OpT*>(ws.dSsnap) + ch * D * D + frag_off<D>(d0 + l16, j0 + 8 * hf), vals);
    }
    // scaled dO slice, transposed into LDS (rows past the end are zero)
    {
        float4v x;
        const int64_t tb = c * CHUNK + 16 * wid + 4 * g4;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (tb + e < T) ? scale * to_f32(cur.dO[e]) : 0.f;
        st4b<OpT>(s_dO + l16 * LDS_U + 16 * wid + 4 * g4, x);
    }
    __syncthreads();

    // dU = A^T dO + Kb dS'   (A^T is upper triangular: rows 16w.. need k >= 16w)
    float4v du = zero4();
    {
        Frag<OpT> fo;
        if (wid < 2) {
            fo.load(s_dO + l16 * LDS_U + 8 * g4);
            mma(cur.at[0], fo, du);
        }
        fo.load(s_dO + l16 * LDS_U + 32 + 8 * g4);
        mma(cur.at[1], fo, du);
#pragma unroll
        for (int kq = 0; kq < D / 32; ++kq) {
            Frag<OpT> fs;
            fs.load(s_dS + l16 * LDS_S + 32 * kq + 8 * g4);
            mma(cur.kb[kq], fs, du);
        }
    }
    if constexpr (CLER) {
        // saved: dU - M^T dE; state update: dU + dE / beta
        const int64_t tb = c * CHUNK + 16 * wid + 4 * g4;
        float4v due;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            due[e] = du[e] - to_f32(cur.mt[e]);
            if (tb + e < T) du[e] += lamj * to_f32(cur.dh[e]) / cur.bt[e];
        }
        st4b<OpT>(s_dUE + l16 * LDS_U + 16 * wid + 4 * g4, due);
    }
    st4b<OpT>(s_dU + l16 * LDS_U + 16 * wid + 4 * g4, du);
    __syncthreads();

    // dU saves: [64][D] rows position (k = column) and [D][64] rows column (k = position)
    const OpT* s_sv = CLER ? s_dUE : s_dU;
    if (tid < 2 * CHUNK) {
        const int grp = tid >> 4, pos0 = 16 * (grp & 3), hf = grp >> 2;
        OpT vals[8];
        lds_column8<LDS_U>(s_sv, 8 * hf, pos0, lane, vals);
        st8(reinterpret_cast<OpT*>(ws.dUsave) + ch * CHUNK * D + frag_off<D>(pos0 + l16, j0 + 8 * hf), vals);
    } else if (tid < 2 * CHUNK + 128) {
        const int t2 = tid - 2 * CHUNK, j = t2 >> 3, pg = t2 & 7;  // column j, positions 8pg..8pg+7
        OpT vals[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vals[e] = s_sv[j * LDS_U + 8 * pg + e];
        st8(reinterpret_cast<OpT*>(ws.dUsaveT) + ch * D * CHUNK + frag_off<CHUNK>(j0 + j, 8 * pg), vals);
    }

    // dS = Diag(gamma) dS' + Qt^T dO - W^T dU
    Frag<OpT> fo0, fo1, fu0, fu1;
    fo0.load(s_dO + l16 * LDS_U + 8 * g4);
    fo1.load(s_dO + l16 * LDS_U + 32 + 8 * g4);
    fu0.load(s_dU + l16 * LDS_U + 8 * g4);
    fu1.load(s_dU + l16 * LDS_U + 32 + 8 * g4);
#pragma unroll
    for (int m = 0; m < SRT; ++m) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dS[m][e] *= cur.gam[m][e];
        mma(cur.qtt[m][0], fo0, dS[m]);
        mma(cur.qtt[m][1], fo1, dS[m]);
        float4v wdu = zero4();
        mma(cur.wt[m][0], fu0, wdu);
        mma(cur.wt[m][1], fu1, wdu);
        dS[m] -= wdu;
        // s_dS was last read before the previous barrier
        st4b<OpT>(s_dS + l16 * LDS_S + wid * (D / 4) + 16 * m + 4 * g4, dS[m]);
    }
    __syncthreads();
}

template <int D, bool IN_F32, bool CLER>
__global__ __launch_bounds__(256) void state_bwd_kernel(int64_t T, int H, int64_t NC, float scale, ChunkWs ws,
                                                        const void* __restrict__ dO, const float* __restrict__ dST,
                                                        float* __restrict__ dS0, ClerBwd cl, ChunkRange cr) {
    using Cfg = BwdCfg<D, IN_F32>;
    using OpT = typename Cfg::OpT;
    constexpr int NSL = Cfg::NSL, SRT = Cfg::SRT, LDS_S = Cfg::LDS_S, LDS_U = Cfg::LDS_U;

    __shared__ __attribute__((aligned(16))) OpT s_dS[Cfg::NS * LDS_S];
    __shared__ __attribute__((aligned(16))) OpT s_dO[Cfg::NS * LDS_U];
    __shared__ __attribute__((aligned(16))) OpT s_dU[Cfg::NS * LDS_U];
    __shared__ __attribute__((aligned(16))) OpT s_dUE[CLER ? Cfg::NS * LDS_U : 8];

    const int64_t nblk = gridDim.x;
    int64_t lid = blockIdx.x;
    if (nblk % 8 == 0) lid = (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
    const int64_t bh = lid / NSL;
    const int j0 = static_cast<int>(lid % NSL) * Cfg::NS;
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh % H);
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const float lamj = (CLER && cl.lam) ? cl.lam[static_cast<int64_t>(h) * D + j0 + l16] : 1.f;

    float4v dS[SRT];
#pragma unroll
    for (int m = 0; m < SRT; ++m) {
        const int d0 = wid * (D / 4) + 16 * m + 4 * g4;
#pragma unroll
        for (int e = 0; e < 4; ++e) dS[m][e] = dST ? dST[(bh * D + d0 + e) * D + j0 + l16] : 0.f;
        st4b<OpT>(s_dS + l16 * LDS_S + d0, dS[m]);
    }
    __syncthreads();

    BwdFrags<D, IN_F32> fa, fb;
    const int64_t clo = cr.lo, chi = cr.lo + cr.n - 1;  // chunks chi down to clo
    if (cr.n > 0) load_bwd<D, IN_F32, CLER>(fa, ws, bh * NC + chi, chi, b, T, H, h, dO, j0, wid, lane, cl);
#pragma unroll 1
    for (int64_t c = chi; c >= clo; c -= 2) {
        const int64_t n1 = c - 1 >= clo ? c - 1 : clo;
        load_bwd<D, IN_F32, CLER>(fb, ws, bh * NC + n1, n1, b, T, H, h, dO, j0, wid, lane, cl);
        bwd_step<D, IN_F32, CLER>(fa, c, T, bh, NC, j0, wid, lane, scale, lamj, ws, dS, s_dS, s_dO, s_dU, s_dUE);
        if (c - 1 < clo) break;
        const int64_t n2 = c - 2 >= clo ? c - 2 : clo;
        load_bwd<D, IN_F32, CLER>(fa, ws, bh * NC + n2, n2, b, T, H, h, dO, j0, wid, lane, cl);
        bwd_step<D, IN_F32, CLER>(fb, c - 1, T, bh, NC, j0, wid, lane, scale, lamj, ws, dS, s_dS, s_dO, s_dU,
                                  s_dUE);
    }

    if (dS0) {
#pragma unroll
        for (int m = 0; m < SRT; ++m) {
            const int d0 = wid * (D / 4) + 16 * m + 4 * g4;
#pragma unroll
            for (int e = 0; e < 4; ++e) dS0[(bh * D + d0 + e) * D + j0 + l16] = dS[m][e];
        }
    }
}

// ---------------------------------------------------------------------------
// LDS-staged variant for fp16 operands.  A workgroup carries NSW slices of one
// head: waves 4 s .. 4 s + 3 run slice s, and the last four waves copy chunk
// c-1's operands (A^T, Kb, Qt^T, W^T, gamma and the slices' dO rows) from
// global memory straight into the LDS buffer that chunk c+1 used, while the
// compute waves run chunk c from the other buffer; they also pull chunk c-PF
// into the L2.  The slices share the staged operands, so each chunk is staged
// D / (16 NSW) times instead of D / 16, and the pass occupies that many CUs per
// head, which leaves the rest to the gradient kernels that run beside it (a
// wave that ran several slices would lengthen the serial step).  The dO
// fragments are built directly from the staged rows, so a step needs only two
// barriers (after dU, after dS).
// ---------------------------------------------------------------------------

// The forward's operands A, Kb^T, Qt and W are staged as stored (fragment
// order); the step reads the fragments of their transposes A^T, Kb, Qt^T and
// W^T as column pieces with transposed LDS reads.
template <int D, bool CLER, int NSW>
struct BwdStage {
    static constexpr int MAT = CHUNK * D * 2;   // [64][D] or [D][64] fp16
    static constexpr int A = 0;                 // A [64][64]
    static constexpr int KBT = A + CHUNK * CHUNK * 2;  // Kb^T [D][64]
    static constexpr int QT = KBT + MAT;        // Qt [64][D]
    static constexpr int W = QT + MAT;          // W [64][D]
    static constexpr int DO = W + MAT;          // dO rows of each slice: NSW x [64][16] in the input dtype (bf16)
    static constexpr int GAM = DO + NSW * 2048; // D fp32 in a 1 KiB slot
    static constexpr int DH = GAM + 1024;       // error routing: dh rows of each slice, like dO
    static constexpr int BT = DH + NSW * 2048;  // error routing: the chunk's 64 betas (1 KiB slot)
    static constexpr int MT = BT + 1024;        // error routing: M^T dE rows of each slice (fp16)
    static constexpr int BYTES = CLER ? MT + NSW * 2048 : GAM + 1024;
    static constexpr int NSL = D / 16;
    static constexpr int NL = (CHUNK * CHUNK * 2 + 3 * MAT) / NSL / 128 + 1;  // lines touched per chunk and slice
    static constexpr int NT = (NL + 63) / 64;
};

// PART 0: A, the dO rows of the NSW slices from column j0 on, gamma (and the
// epilogue's dh rows and betas); PART 1: Kb^T; PART 2: Qt; PART 3: W.
template <int D, bool CLER, int NSW, int PART>
__device__ __forceinline__ void stage_bwd(lds_char* dst, const ChunkWs& ws, int64_t ch, int64_t c, int64_t b,
                                          int64_t T, int H, int h, const void* dO, int j0, int lane,
                                          const ClerBwd& cl) {
    using L = BwdStage<D, CLER, NSW>;
    if constexpr (PART == 1) {
        copy_block_to_lds<L::MAT / 1024>(static_cast<const char*>(ws.KbT) + ch * L::MAT, dst + L::KBT, lane);
    } else if constexpr (PART == 2) {
        copy_block_to_lds<L::MAT / 1024>(static_cast<const char*>(ws.Qt) + ch * L::MAT, dst + L::QT, lane);
    } else if constexpr (PART == 3) {
        copy_block_to_lds<L::MAT / 1024>(static_cast<const char*>(ws.W) + ch * L::MAT, dst + L::W, lane);
    } else {
        copy_block_to_lds<CHUNK * CHUNK * 2 / 1024>(static_cast<const char*>(ws.A) + ch * CHUNK * CHUNK * 2,
                                                    dst + L::A, lane);
        // dO rows: position pos = 32 i + lane / 2, half lane % 2 of the slice's 16
        // columns (rows past the end re-read the last token; they are zeroed at use)
#pragma unroll
        for (int sl = 0; sl < NSW; ++sl) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int64_t t0 = c * CHUNK + 32 * i + (lane >> 1);
                const int64_t t = t0 < T ? t0 : T - 1;
                const char* src =
                    static_cast<const char*>(dO) + (((b * T + t) * H + h) * D + j0 + 16 * sl + 8 * (lane & 1)) * 2;
                copy16_to_lds(src, dst + L::DO + sl * 2048 + i * 1024);
            }
        }
        const char* G = reinterpret_cast<const char*>(ws.gam + ch * D);
        copy16_to_lds(G + (lane < D / 4 ? lane : 0) * 16, dst + L::GAM);
        if constexpr (CLER) {
#pragma unroll
            for (int sl = 0; sl < NSW; ++sl) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int64_t t0 = c * CHUNK + 32 * i + (lane >> 1);
                    const int64_t t = t0 < T ? t0 : T - 1;
                    const char* src = static_cast<const char*>(cl.dh) +
                                      (((b * T + t) * H + h) * D + j0 + 16 * sl + 8 * (lane & 1)) * 2;
                    copy16_to_lds(src, dst + L::DH + sl * 2048 + i * 1024);
                }
            }
            const int64_t t0 = c * CHUNK + lane;
            const int64_t t = t0 < T ? t0 : T - 1;
            copy4_to_lds(cl.beta + (b * T + t) * H + h, dst + L::BT);
#pragma unroll
            for (int sl = 0; sl < NSW; ++sl) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int pos = 32 * i + (lane >> 1);
                    const char* src = static_cast<const char*>(ws.Mt) +
                                      ((ch * CHUNK + pos) * D + j0 + 16 * sl + 8 * (lane & 1)) * 2;
                    copy16_to_lds(src, dst + L::MT + sl * 2048 + i * 1024);
                }
            }
        }
    }
}

// Loader wave `part` (0..3) copies its share of chunk ch.
template <int D, bool CLER, int NSW>
__device__ __forceinline__ void stage_bwd_part(int part, lds_char* dst, const ChunkWs& ws, int64_t ch, int64_t c,
                                               int64_t b, int64_t T, int H, int h, const void* dO, int j0, int lane,
                                               const ClerBwd& cl) {
    if (part == 0) stage_bwd<D, CLER, NSW, 0>(dst, ws, ch, c, b, T, H, h, dO, j0, lane, cl);
    else if (part == 1) stage_bwd<D, CLER, NSW, 1>(dst, ws, ch, c, b, T, H, h, dO, j0, lane, cl);
    else if (part == 2) stage_bwd<D, CLER, NSW, 2>(dst, ws, ch, c, b, T, H, h, dO, j0, lane, cl);
    else stage_bwd<D, CLER, NSW, 3>(dst, ws, ch, c, b, T, H, h, dO, j0, lane, cl);
}

template <int D>
__device__ __forceinline__ void touch_bwd(lds_char* dummy, const ChunkWs& ws, int64_t ch, int slice, int lane) {
    using L = BwdStage<D, false, 1>;
    constexpr int AL = CHUNK * CHUNK * 2 / L::NSL / 128, QL = L::MAT / L::NSL / 128;
#pragma unroll
    for (int i = 0; i < L::NT; ++i) {
        const int Lr = lane + 64 * i;
        const char* addr;
        if (Lr < AL) addr = static_cast<const char*>(ws.A) + ch * CHUNK * CHUNK * 2 + (slice * AL + Lr) * 128;
        else if (Lr < AL + QL) addr = static_cast<const char*>(ws.KbT) + ch * L::MAT + (slice * QL + Lr - AL) * 128;
        else if (Lr < AL + 2 * QL)
            addr = static_cast<const char*>(ws.Qt) + ch * L::MAT + (slice * QL + Lr - AL - QL) * 128;
        else if (Lr < AL + 3 * QL)
            addr = static_cast<const char*>(ws.W) + ch * L::MAT + (slice * QL + Lr - AL - 2 * QL) * 128;
        else addr = reinterpret_cast<const char*>(ws.gam + ch * D) + (slice % (D * 4 / 128)) * 128;
        copy4_to_lds(addr, dummy + i * 256);
    }
}

template <int D, bool CLER, int NSW>
__global__ __launch_bounds__(64 * (4 * NSW + 4)) void state_bwd_lds_kernel(int64_t T, int H, int64_t NC, float scale,
                                                                           ChunkWs ws, const void* __restrict__ dO,
                                                                           const float* __restrict__ dST,
                                                                           float* __restrict__ dS0, ClerBwd cl,
                                                                           ChunkRange cr) {
    using Cfg = BwdCfg<D, false>;
    using OpT = _Float16;
    using L = BwdStage<D, CLER, NSW>;
    using LT = BwdStage<D, false, 1>;
    constexpr int NSL = Cfg::NSL, SRT = Cfg::SRT, LDS_S = Cfg::LDS_S, LDS_U = Cfg::LDS_U;
    constexpr int NG = NSL / NSW;  // workgroups per head
    constexpr int PF = 8;
    static_assert(NSL % NSW == 0, "slices per workgroup");

    __shared__ __attribute__((aligned(16))) OpT s_dS[NSW][Cfg::NS * LDS_S];
    __shared__ __attribute__((aligned(16))) OpT s_dU[NSW][Cfg::NS * LDS_U];
    __shared__ __attribute__((aligned(16))) OpT s_dUE[NSW][CLER ? Cfg::NS * LDS_U : 8];
    __shared__ __attribute__((aligned(1024))) char stage[2][L::BYTES];
    __shared__ __attribute__((aligned(16))) char dummy[LT::NT * 256];

    const int64_t nblk = gridDim.x;
    int64_t lid = blockIdx.x;
    if (nblk % 8 == 0) lid = (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
    const int64_t bh = lid / NG;
    const int grp = static_cast<int>(lid % NG);
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh % H);
    const int tid = threadIdx.x, lane = tid & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    lds_char* const sbuf = (lds_char*)&stage[0][0];
    lds_char* const sdummy = (lds_char*)&dummy[0];
    const int64_t clo = cr.lo, chi = cr.lo + cr.n - 1;  // chunks chi down to clo

    if (tid >= 256 * NSW) {
        // Loaders: chunk c-1 goes into the buffer chunk c+1 used (free since the
        // end of that step).  Four waves each copy one part (A, dO and gamma;
        // Kb^T; Qt; W), so four times as many copies are in flight as with
        // one; the first also warms the L2 (the lines of this group's slices).
        const int part = (tid >> 6) - 4 * NSW;
        const bool w4 = part == 0;
        const int jg = grp * NSW * 16;
        if (cr.n > 0) stage_bwd_part<D, CLER, NSW>(part, sbuf, ws, bh * NC + chi, chi, b, T, H, h, dO, jg, lane, cl);
        if (w4) {
#pragma unroll 1
            for (int64_t c = chi - 1; c >= 0 && c > chi - PF; --c)
#pragma unroll
                for (int sl = 0; sl < NSW; ++sl) touch_bwd<D>(sdummy, ws, bh * NC + c, grp * NSW + sl, lane);
        }
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        int nb = 1;  // buffer of chunk c-1
#pragma unroll 1
        for (int64_t c = chi; c >= clo; --c) {
            const bool st = c >= clo + 1, tpf = w4 && c - PF >= 0;
            if (st)
                stage_bwd_part<D, CLER, NSW>(part, sbuf + nb * L::BYTES, ws, bh * NC + c - 1, c - 1, b, T, H, h, dO,
                                             jg, lane, cl);
            if (tpf) {
#pragma unroll
                for (int sl = 0; sl < NSW; ++sl) touch_bwd<D>(sdummy, ws, bh * NC + c - PF, grp * NSW + sl, lane);
            }
            __builtin_amdgcn_s_barrier();
            // chunk c-1 must have landed; only this step's touches may stay in flight
            if (tpf) wait_vmcnt<NSW * LT::NT>();
            else wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            nb ^= 1;
        }
        return;
    }

    // compute waves: slice sl of the group, wave wid (0..3) within the slice
    const int sl = tid >> 8, wid = (tid >> 6) & 3, stid = tid & 255;
    const int j0 = (grp * NSW + sl) * Cfg::NS;
    OpT* const sdS = s_dS[sl];
    OpT* const sdU = s_dU[sl];
    OpT* const sdUE = s_dUE[sl];
    const float lamj = (CLER && cl.lam) ? cl.lam[static_cast<int64_t>(h) * D + j0 + l16] : 1.f;
    float4v dS[SRT];
#pragma unroll
    for (int m = 0; m < SRT; ++m) {
        const int d0 = wid * (D / 4) + 16 * m + 4 * g4;
#pragma unroll
        for (int e = 0; e < 4; ++e) dS[m][e] = dST ? dST[(bh * D + d0 + e) * D + j0 + l16] : 0.f;
        st4b<OpT>(sdS + l16 * LDS_S + d0, dS[m]);
    }
    __syncthreads();

    int cb = 0;
#pragma unroll 1
    for (int64_t c = chi; c >= clo; --c) {
        const lds_char* src = sbuf + cb * L::BYTES;
        cb ^= 1;
        const int64_t ch = bh * NC + c;
        // operand fragments of this wave for dU (those for dS are read once the
        // dU products are issued)
        // fragment whose lane holds rows r0 + 8 g4 .. +7 of column c0 + l16 of a
        // fragment-order array staged at byte offset `at_` (K its row length)
        const auto colfrag = [&](int at_, int K, int r0, int c0) {
            typedef const __attribute__((address_space(3))) _Float16* lds_f16;
            _Float16 x[8];
            if (K == CHUNK)
                lds_column8_at(reinterpret_cast<lds_f16>(src + at_), r0 + 8 * g4, c0, lane,
                               [](int r, int c) { return frag_off<CHUNK>(r, c); }, x);
            else
                lds_column8_at(reinterpret_cast<lds_f16>(src + at_), r0 + 8 * g4, c0, lane,
                               [](int r, int c) { return frag_off<D>(r, c); }, x);
            Frag<OpT> f;
#pragma unroll
            for (int e = 0; e < 8; ++e) f.v[e] = x[e];
            return f;
        };
        Frag<OpT> at[2], kb[D / 32], qtt[SRT][2], wt[SRT][2];
        float gam[SRT][4];
        // A^T (rows 16 wid + l16, k = position) and Kb (rows position, k = d):
        // column pieces of A and Kb^T
        at[0] = colfrag(L::A, CHUNK, 0, 16 * wid);
        at[1] = colfrag(L::A, CHUNK, 32, 16 * wid);
#pragma unroll
        for (int kq = 0; kq < D / 32; ++kq) kb[kq] = colfrag(L::KBT, CHUNK, 32 * kq, 16 * wid);
        // dO fragments (B operand, k = position): column j0 + l16, positions
        // 32 kq + 8 g4 + e, scaled; rows past the end are zero
        // (all sixteen values are read before any is masked: a select on each
        // read would become a branch that waits for every LDS read before it)
        const int64_t nvc = T - c * CHUNK;  // positions of this chunk inside the sequence
        Frag<OpT> fo[2];
        {
            const __attribute__((address_space(3))) bf16_t* dos =
                reinterpret_cast<const __attribute__((address_space(3))) bf16_t*>(src + L::DO + sl * 2048);
            bf16_t raw[2][8];
#pragma unroll
            for (int kq = 0; kq < 2; ++kq)
                lds_column8_at(dos, 32 * kq + 8 * g4, 0, lane, [](int r, int c) { return r * 16 + c; }, raw[kq]);
            asm volatile("" ::: "memory");
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = scale * bf16_to_f32(raw[kq][e]);
                    fo[kq].v[e] = from_f32<_Float16>(32 * kq + 8 * g4 + e < nvc ? x : 0.f);
                }
            }
        }

        // dU = A^T dO + Kb dS'   (A^T's lower blocks are zero)
        float4v du = zero4();
        mma(at[0], fo[0], du);
        mma(at[1], fo[1], du);
#pragma unroll
        for (int kq = 0; kq < D / 32; ++kq) {
            Frag<OpT> fs;
            fs.load(sdS + l16 * LDS_S + 32 * kq + 8 * g4);
            mma(kb[kq], fs, du);
        }
        if constexpr (CLER) {
            // saved: dU - M^T dE; state update: dU + lam dh / beta (rows 16 wid + 4 g4 + e)
            const __attribute__((address_space(3))) bf16_t* dhs =
                reinterpret_cast<const __attribute__((address_space(3))) bf16_t*>(src + L::DH + sl * 2048);
            const __attribute__((address_space(3))) _Float16* mts =
                reinterpret_cast<const __attribute__((address_space(3))) _Float16*>(src + L::MT + sl * 2048);
            const float4v bt =
                *reinterpret_cast<const __attribute__((address_space(3))) float4v*>(src + L::BT + (16 * wid + 4 * g4) * 4);
            float4v due;
            bf16_t dhr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) dhr[e] = dhs[(16 * wid + 4 * g4 + e) * 16 + l16];
            asm volatile("" ::: "memory");
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int pos = 16 * wid + 4 * g4 + e;
                due[e] = du[e] - static_cast<float>(mts[pos * 16 + l16]);
                if (pos < nvc) du[e] += lamj * bf16_to_f32(dhr[e]) / bt[e];
            }
            st4b<OpT>(sdUE + l16 * LDS_U + 16 * wid + 4 * g4, due);
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int m = 0; m < SRT; ++m) {
            const int rt = wid * (D / 64) + m;
            // Qt^T and W^T (rows d = 16 rt + l16, k = position): column pieces of Qt and W
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                qtt[m][kq] = colfrag(L::QT, D, 32 * kq, 16 * rt);
                wt[m][kq] = colfrag(L::W, D, 32 * kq, 16 * rt);
            }
            const float4v g = *reinterpret_cast<const __attribute__((address_space(3))) float4v*>(src + L::GAM + (16 * rt + 4 * g4) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) gam[m][e] = g[e];
        }
        st4b<OpT>(sdU + l16 * LDS_U + 16 * wid + 4 * g4, du);
        __syncthreads();

        // dU save: [64][D] rows position (k = column); the gradient kernel reads
        // its transpose from the same copy
        {
            const OpT* s_sv = CLER ? sdUE : sdU;
            const int t = stid;
            if (t < 2 * CHUNK) {
                // each 16-lane group 16 positions and 8 of the columns
                const int grp = t >> 4, pos0 = 16 * (grp & 3), hf = grp >> 2;
                OpT vals[8];
                lds_column8<LDS_U>(s_sv, 8 * hf, pos0, lane, vals);
                st8(reinterpret_cast<OpT*>(ws.dUsave) + ch * CHUNK * D + frag_off<D>(pos0 + l16, j0 + 8 * hf), vals);
            }
        }
        // chunk-end gradient dS' (rows d, k = column): each wave saves the rows
        // it owns before it overwrites them below
        {
            constexpr int RW = D / 4, RG = RW / 16;
            if (g4 < 2 * RG) {  // each 16-lane group 16 rows and 8 of the columns
                const int d0 = RW * wid + 16 * (g4 % RG), hf = g4 / RG;
                OpT vals[8];
                lds_column8<LDS_S>(sdS, 8 * hf, d0, lane, vals);
                st8(reinterpret_cast<OpT*>(ws.dSsnap) + ch * D * D + frag_off<D>(d0 + l16, j0 + 8 * hf), vals);
            }
        }

        // dS = Diag(gamma) dS' + Qt^T dO - W^T dU
        Frag<OpT> fu0, fu1;
        fu0.load(sdU + l16 * LDS_U + 8 * g4);
        fu1.load(sdU + l16 * LDS_U + 32 + 8 * g4);
#pragma unroll
        for (int m = 0; m < SRT; ++m) {
#pragma unroll
            for (int e = 0; e < 4; ++e) dS[m][e] *= gam[m][e];
            mma(qtt[m][0], fo[0], dS[m]);
            mma(qtt[m][1], fo[1], dS[m]);
            float4v wdu = zero4();
            mma(wt[m][0], fu0, wdu);
            mma(wt[m][1], fu1, wdu);
            dS[m] -= wdu;
            st4b<OpT>(sdS + l16 * LDS_S + wid * (D / 4) + 16 * m + 4 * g4, dS[m]);
        }
        __syncthreads();
    }

    if (dS0) {
#pragma unroll
        for (int m = 0; m < SRT; ++m) {
            const int d0 = wid * (D / 4) + 16 * m + 4 * g4;
#pragma unroll
            for (int e = 0; e < 4; ++e) dS0[(bh * D + d0 + e) * D + j0 + l16] = dS[m][e];
        }
    }
}

template <int D, bool IN_F32, bool CLER>
static void launch_state_bwd_c(int64_t nblk, int64_t T, int H, int64_t NC, float scale, const ChunkWs& ws,
                               const void* dO, const float* dST, float* dS0, const ClerBwd& cl, bool wide,
                               ChunkRange cr, hipStream_t stream) {
    if constexpr (!IN_F32) {
        if (wide)
            hipLaunchKernelGGL((state_bwd_lds_kernel<D, CLER, 2>), dim3((unsigned)(nblk / 2)), dim3(64 * 12), 0,
                               stream, T, H, NC, scale, ws, dO, dST, dS0, cl, cr);
        else
            hipLaunchKernelGGL((state_bwd_lds_kernel<D, CLER, 1>), dim3((unsigned)nblk), dim3(64 * 8), 0, stream,
                               T, H, NC, scale, ws, dO, dST, dS0, cl, cr);
    } else {
        hipLaunchKernelGGL((state_bwd_kernel<D, IN_F32, CLER>), dim3((unsigned)nblk), dim3(256), 0, stream, T, H,
                           NC, scale, ws, dO, dST, dS0, cl, cr);
    }
}

template <int D, bool IN_F32>
static hipError_t launch_state_bwd_t(int64_t B, int64_t T, int H, int64_t NC, float scale, const ChunkWs& ws,
                                     const void* dO, const float* dST, float* dS0, const ClerBwd& cl, bool wide,
                                     ChunkRange cr, hipStream_t stream) {
    const int64_t nblk = B * H * BwdCfg<D, IN_F32>::NSL;
    if (nblk == 0) return hipSuccess;
    if (cl.dh) launch_state_bwd_c<D, IN_F32, true>(nblk, T, H, NC, scale, ws, dO, dST, dS0, cl, wide, cr, stream);
    else launch_state_bwd_c<D, IN_F32, false>(nblk, T, H, NC, scale, ws, dO, dST, dS0, cl, wide, cr, stream);
    return hipGetLastError();
}

hipError_t launch_state_bwd(int D, bool in_f32, int64_t B, int64_t T, int H, int64_t NC, float scale,
                            const ChunkWs& ws, const void* dO, const float* dST, float* dS0,
                            const void* dh_cler, const float* lam, const float* beta, bool wide, ChunkRange cr,
                            hipStream_t stream) {
    const ClerBwd cl{dh_cler, lam, beta};
#define GDR_SB_ARGS B, T, H, NC, scale, ws, dO, dST, dS0, cl, wide, cr, stream
    if (D == 64) {
        if (in_f32) return launch_state_bwd_t<64, true>(GDR_SB_ARGS);
        return launch_state_bwd_t<64, false>(GDR_SB_ARGS);
    }
    if (in_f32) return launch_state_bwd_t<128, true>(GDR_SB_ARGS);
    return launch_state_bwd_t<128, false>(GDR_SB_ARGS);
#undef GDR_SB_ARGS
}

}  // namespace gdr
