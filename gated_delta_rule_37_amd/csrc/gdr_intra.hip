// gdr_intra.hip -- intra-chunk transform of the chunked gated delta rule.
//
// One workgroup per (batch, head, chunk of 64 tokens).  With S the chunk's start
// state, G_r the in-chunk inclusive sum of log2(alpha) (kept in log space for
// range safety, KDA blog section 7.1) and, row-wise,
//   Kt = K*2^G, Kh = K*2^-G, Qt = Q*2^G, Kb = K*2^(G_last - G),
// unrolling the token recurrence over the chunk gives
//   U = T (V - Kt S),  T = (I + L)^-1 diag(beta),
//   L = strict_tril(diag(beta) Kt Kh^T),
//   O = Qt S + A U,    A = tril(Qt Kh^T),
//   S_next = Diag(2^G_last) S + Kb^T U.
// This kernel computes everything that does not depend on S -- the rank-1
// updates of the chunk gathered into one triangular solve plus dense products
// (the "UT transform" of the KDA blog, section 6.2) -- and writes, per chunk,
//   W = T Kt, Ut = T V, Qt, Kb^T, A and gamma = 2^G_last
// for the sequential state pass.  The optional CLVR epilogue (h += lam * v) is
// fused here because this kernel already reads v.  Every operand of the state
// pass is written in fragment order (see gdr_common.hpp) so that the
// sequential kernel reads it with fully coalesced loads.  In backward mode it writes
// instead the operands the reverse state pass and the gradient kernel need:
// W, Ut, Kb^T, gamma, Qt, A, N = (I + L)^-1 and P in fp32; the reverse pass
// reads the transposes of Qt, A, Kb^T and W with transposed LDS reads (fp32
// operands: A^T, Kb, Qt^T and W^T are stored instead of Qt and A).
//
// Thread layout: 4*D threads; thread (channel c, part p) owns rows 16p..16p+15
// of channel c for the element-wise work, i.e. exactly the 16-row block p.
//
// Range handling for the channel gate (Kimi Delta Attention).  The pair factor
// 2^(G_r - G_i) (r >= i) is <= 1, but Kt Kh^T written naively overflows for
// strong gates.  Block row R uses the reference value ref(R) = G at the last
// row before block R, so that
//   row operand    Kq_r = k_r 2^(G_r - ref(R))   <= 1
//   column operand Kh_i = k_i 2^(ref(R) - G_i)  <= 1 for i before block R,
// and only the 16x16 diagonal block has column factors >= 1 (bounded by the
// block's own decay range rho).  When rho exceeds what the operand precision
// can carry, that diagonal block is recomputed exactly on the vector ALUs from
// running products of alpha (no exponentials, no overflow).  The exponentials
// themselves are formed as 2^G and 2^-G once per element times per-channel
// scalars when the chunk's total decay fits the fp32 exponent range, and pair
// by pair otherwise.  For the scalar gate the factor does not depend on the
// channel, so K K^T and Q K^T are taken on the raw inputs and the decay mask is
// applied afterwards in fp32.
#include "gdr_common.hpp"
#include "gdr_launch.hpp"

#include <type_traits>

namespace gdr {

template <int D, int GATE, bool IN_F32>
struct IntraLayout {
    using OpT = typename std::conditional<IN_F32, float, _Float16>::type;
    static constexpr int OPB = sizeof(OpT);
    static constexpr int PAD = 16 / OPB;  // one 16-byte granule per row: conflict-free fragment reads
    static constexpr int LDR = D + PAD;   // row stride of [64][D] arrays
    static constexpr int LDC = CHUNK + PAD;  // row stride of [D][64] and [64][64] operand arrays
    static constexpr int NT = 4 * D;         // threads
    static constexpr int NW = NT / WAVE;     // waves
    static constexpr int RPP = 16;           // rows per thread (one 16-row block)
    // phase 1-2: Kq, Qq ([64][LDR]) and Kh: [64][LDR], or for the channel gate
    // with fp16 operands at d = 128 (KH4) the column operands of all four block
    // rows, R = 0..3 holding rows 0 .. 16R+15 from row 8R(R+1) on (160 rows).
    // (At d = 64 the larger buffer would stop two workgroups sharing a CU; with
    // fp32 operands it does not fit.)
    static constexpr bool KH4 = GATE == GATE_CHANNEL && !IN_F32 && D == 128;
    static constexpr int KQ = 0;
    static constexpr int QQ = KQ + CHUNK * LDR * OPB;
    static constexpr int KH = QQ + CHUNK * LDR * OPB;
    static constexpr int KH_ROWS = KH4 ? 160 : CHUNK;
    static constexpr int END12 = KH + KH_ROWS * LDR * OPB;
    // phase 3-4: Kt^T, V^T ([D][LDC]), P/L/T, N
    static constexpr int KTT = 0;
    static constexpr int VT = KTT + D * LDC * OPB;
    static constexpr int PL = VT + D * LDC * OPB;
    static constexpr int PL_BYTES = (CHUNK * CHUNK * 4 > CHUNK * LDC * OPB) ? CHUNK * CHUNK * 4 : CHUNK * LDC * OPB;
    // N (and, during phase 2, the fp32 P staging) must not overlap phase 1-2 buffers
    static constexpr int NM = (PL + PL_BYTES > END12) ? PL + PL_BYTES : END12;
    static constexpr int END34 = NM + CHUNK * CHUNK * 4;
    static constexpr int BASE_BYTES = END12 > END34 ? END12 : END34;
    // fp16 operands: Qt (fragment order) and the updated h rows are assembled
    // in LDS and written out with full 16-byte stores
    static constexpr bool STAGE = !IN_F32;
    static constexpr int QTS = BASE_BYTES;
    static constexpr int HS = QTS + (STAGE ? CHUNK * D * OPB : 0);
    static constexpr int BYTES = HS + (STAGE ? CHUNK * D * 2 : 0);
    // operand-precision limit on the in-block decay range (log2 units)
    static constexpr float RHO_MAX = IN_F32 ? 100.f : 8.f;
    // chunk decay beyond which 2^G or 2^-G leaves the fp32 range (log2 units)
    static constexpr float WIDE_MAX = 120.f;
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

// MODE 0: the forward's operands (and CLVR); 1: the operands of the recomputing
// backward; 2: both, so that a training forward leaves everything its backward needs.
// PRO: the prologue (pro = 1 or 2 selects the alpha activation).
template <int D, int GATE, bool IN_F32, int MODE, bool PRO>
__global__ __launch_bounds__(4 * D) void intra_kernel(int64_t T, int H, int64_t NC,
                                                      const void* __restrict__ q_,
                                                      const void* __restrict__ k_,
                                                      const void* __restrict__ v_,
                                                      const float* __restrict__ beta,
                                                      const float* __restrict__ alpha,
                                                      void* __restrict__ h_, const float* __restrict__ lam,
                                                      ChunkWs ws, int pro, ChunkRange cr) {
    constexpr bool FO = MODE != 1;  // forward operands: Qt, A
    constexpr bool BWD = MODE != 0; // backward operands: N, P (and the prologue's norms)
    // Qt and A: the forward's operands, and with fp16 operands also the reverse
    // pass's, which reads their transposes (and Kb, W^T) with transposed LDS
    // reads; fp32 operands store those transposes (TR) for the reverse pass
    constexpr bool QA = FO || (BWD && !IN_F32);
    constexpr bool TR = BWD && IN_F32;
    using L = IntraLayout<D, GATE, IN_F32>;
    using OpT = typename L::OpT;
    using InT = typename InType<IN_F32>::T;
    constexpr int NT = L::NT, NW = L::NW, RPP = L::RPP, LDR = L::LDR, LDC = L::LDC;

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    __shared__ float s_tot[4][D];  // per-block sums of log2(alpha), then block-end values
    __shared__ float s_gs[CHUNK];  // scalar-gate G per row
    __shared__ float s_beta[CHUNK];
    __shared__ float s_red[NW][2];
    __shared__ float s_nrm[NW * 2 * L::RPP];  // prologue: row-norm partials

    OpT* Kq = reinterpret_cast<OpT*>(smem + L::KQ);
    OpT* Qq = reinterpret_cast<OpT*>(smem + L::QQ);
    OpT* Kh = reinterpret_cast<OpT*>(smem + L::KH);
    OpT* QtS = reinterpret_cast<OpT*>(smem + L::QTS);  // staged output (fp16 operands only)
    OpT* KtT = reinterpret_cast<OpT*>(smem + L::KTT);
    OpT* VT = reinterpret_cast<OpT*>(smem + L::VT);
    float* Pm = reinterpret_cast<float*>(smem + L::PL);
    OpT* Tm = reinterpret_cast<OpT*>(smem + L::PL);
    float* Nm = reinterpret_cast<float*>(smem + L::NM);

    int64_t bh, c;
    range_block(cr, bh, c);
    const int64_t ch = bh * NC + c;
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh % H);
    const int64_t t0 = c * CHUNK;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int cc = tid % D, part = tid / D, r0 = part * RPP;
    const int l16 = lane & 15, g4 = lane >> 4;

    const InT* q = reinterpret_cast<const InT*>(q_);
    const InT* k = reinterpret_cast<const InT*>(k_);
    const InT* v = reinterpret_cast<const InT*>(v_);
    InT* hh = reinterpret_cast<InT*>(h_);
    InT* HS = reinterpret_cast<InT*>(smem + L::HS);
    const int64_t tokstride = static_cast<int64_t>(H) * D;
    const int64_t base = ((b * T + t0) * H + h) * D;  // element (row 0, channel 0) of this chunk
    const int64_t nvalid64 = T - t0;
    const int nvalid = nvalid64 < CHUNK ? static_cast<int>(nvalid64) : CHUNK;

    // ---------------- phase 1: loads ----------------
    // Every global load of the chunk is issued here, back to back.  Rows past the
    // end of the sequence read the last valid row (always in bounds) and are
    // zeroed afterwards, so the loads carry no branches.
    float G[RPP], kk[RPP], vv[RPP], qq[RPP];
    InT hv[RPP];
#pragma unroll
    for (int j = 0; j < RPP; ++j) {
        const int r = r0 + j;
        const int64_t e = base + (r < nvalid ? r : nvalid - 1) * tokstride + cc;
        kk[j] = to_f32(k[e]);
        qq[j] = to_f32(q[e]);
        vv[j] = to_f32(v[e]);
        if constexpr (GATE == GATE_CHANNEL) G[j] = alpha[e];
        else G[j] = 0.f;
    }
    if (hh) {
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            const int r = r0 + j;
            hv[j] = hh[base + (r < nvalid ? r : nvalid - 1) * tokstride + cc];
        }
    }
    if (tid < CHUNK) {
        const bool ok = tid < nvalid;
        const int64_t tok = (b * T + t0 + (ok ? tid : nvalid - 1)) * H + h;
        float bt = beta[tok];
        if constexpr (PRO) {
            // prologue: beta arrives as a logit; the activated value is kept for
            // the later kernels
            bt = sigmoid_fast(bt);
            if (ok) ws.Bact[tok] = bt;
        }
        s_beta[tid] = ok ? bt : 0.f;
        if constexpr (GATE == GATE_SCALAR) {
            const float at = alpha[tok];
            float g = ok ? (PRO ? log2_alpha_logit(at, pro) : log2_fast(at)) : 0.f;
            s_gs[tid] = chunk_prefix_sum(g);
        }
    }
#pragma unroll
    for (int j = 0; j < RPP; ++j) {
        const bool ok = r0 + j < nvalid;
        kk[j] = ok ? kk[j] : 0.f;
        qq[j] = ok ? qq[j] : 0.f;
        vv[j] = ok ? vv[j] : 0.f;
        if constexpr (GATE == GATE_CHANNEL) G[j] = ok ? (PRO ? log2_alpha_logit(G[j], pro) : log2_fast(G[j])) : 0.f;
    }
    if constexpr (PRO) {
        // prologue: q and k rows divided by their L2 norms (sums over the D
        // threads of this part); the backward kernels get the reciprocal norms
        static_assert(2 * RPP == 32, "32 row sums per thread");
        float nrm[2 * RPP];
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            nrm[j] = qq[j] * qq[j];
            nrm[RPP + j] = kk[j] * kk[j];
        }
        part_row_sums32<D>(nrm, s_nrm);
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            const float rq = recip_norm(nrm[j]), rk = recip_norm(nrm[RPP + j]);
            qq[j] *= fabsf(rq);
            kk[j] *= fabsf(rk);
            if constexpr (BWD) {
                const int r = r0 + j;
                if (cc == 0 && r < nvalid) {
                    const int64_t tok = (b * T + t0 + r) * H + h;
                    ws.rq[tok] = rq;
                    ws.rk[tok] = rk;
                }
            }
        }
    }
    if constexpr (GATE == GATE_CHANNEL) {
#pragma unroll
        for (int j = 1; j < RPP; ++j) G[j] += G[j - 1];
        s_tot[part][cc] = G[RPP - 1];
    }
    __syncthreads();

    // ---------------- gate totals, block references, range flags ----------------
    float carry = 0.f, glast = 0.f;  // G before this thread's block, G at the chunk end
    if constexpr (GATE == GATE_CHANNEL) {
        float t[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) t[p] = s_tot[p][cc];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            carry += (p < part) ? t[p] : 0.f;
            glast += t[p];
        }
#pragma unroll
        for (int j = 0; j < RPP; ++j) G[j] += carry;
    } else if constexpr (GATE == GATE_SCALAR) {
#pragma unroll
        for (int j = 0; j < RPP; ++j) G[j] = s_gs[r0 + j];
        glast = s_gs[CHUNK - 1];
    }
    int flags = 0;      // bit R: diagonal block R needs the exact path
    bool wide = false;  // 2^G or 2^-G would leave the fp32 range somewhere in the chunk
    // (scalar gate: one decay for every channel, so the chunk's own total decides;
    // its in-chunk pair factors are formed from G differences and never overflow)
    if constexpr (GATE == GATE_SCALAR) wide = !(-glast <= L::WIDE_MAX);  // NaN-safe
    if constexpr (GATE == GATE_CHANNEL) {
        // each wave holds one block (part) for 64 channels
        const float rho = wave_max(carry - G[RPP - 1]);
        const float span = wave_max(-glast);
        if (lane == 0) {
            s_red[wid][0] = rho;
            s_red[wid][1] = span;
        }
    }
    __syncthreads();  // s_tot is reused below for the block-end values
    if constexpr (GATE == GATE_CHANNEL) {
        s_tot[part][cc] = G[RPP - 1];  // G at the last row of block `part`
        constexpr int WPB = D / WAVE;  // waves per block
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            float rho = s_red[R * WPB][0], span = s_red[R * WPB][1];
#pragma unroll
            for (int w = 1; w < WPB; ++w) {
                rho = fmaxf(rho, s_red[R * WPB + w][0]);
                span = fmaxf(span, s_red[R * WPB + w][1]);
            }
            if (!(rho <= L::RHO_MAX)) flags |= 1 << R;  // NaN-safe
            if (!(span <= L::WIDE_MAX)) wide = true;
        }
    }

    // ---------------- element-wise outputs ----------------
    // Ei[j] = 2^-G (only on the narrow-range path); used again for Kh below
    float E[RPP], Ei[RPP];
    {
        OpT* Qt_g = reinterpret_cast<OpT*>(ws.Qt) + ch * CHUNK * D;
        OpT* KbT_g = reinterpret_cast<OpT*>(ws.KbT) + ch * D * CHUNK;
        float kb[RPP];
        const float egl = exp2_fast(glast);
        const float eref = exp2_fast(-carry);
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            const int r = r0 + j;
            float fq;  // 2^(G_r - ref(R)) for the row operands
            if (!wide) {
                E[j] = exp2_fast(G[j]);
                Ei[j] = exp2_fast(-G[j]);
                kb[j] = kk[j] * (Ei[j] * egl);
                fq = E[j] * eref;
            } else {
                E[j] = exp2_fast(G[j]);
                Ei[j] = 0.f;
                kb[j] = kk[j] * exp2_fast(glast - G[j]);
                fq = exp2_fast(G[j] - carry);
            }
            if constexpr (QA) {
                if constexpr (L::STAGE) QtS[frag_off<D>(r, cc)] = from_f32<OpT>(qq[j] * E[j]);
                else Qt_g[frag_off<D>(r, cc)] = from_f32<OpT>(qq[j] * E[j]);
            }
            if constexpr (GATE == GATE_CHANNEL) {
                Kq[r * LDR + cc] = from_f32<OpT>(kk[j] * fq);
                Qq[r * LDR + cc] = from_f32<OpT>(qq[j] * fq);
            } else {
                Kq[r * LDR + cc] = from_f32<OpT>(kk[j]);
                Qq[r * LDR + cc] = from_f32<OpT>(qq[j]);
                Kh[r * LDR + cc] = from_f32<OpT>(kk[j]);
            }
            if constexpr (TR) {
                OpT* Kb_g = reinterpret_cast<OpT*>(ws.Kb) + ch * CHUNK * D;
                Kb_g[frag_off<D>(r, cc)] = from_f32<OpT>(kb[j]);
            }
        }
        // Kb^T is the A operand of Kb^T U (rows d, k = position): two runs of 8
        store_run<OpT, 8>(KbT_g + frag_off<CHUNK>(cc, r0), kb);
        store_run<OpT, 8>(KbT_g + frag_off<CHUNK>(cc, r0 + 8), kb + 8);
        if constexpr (TR) {
            float qt[RPP];
#pragma unroll
            for (int j = 0; j < RPP; ++j) qt[j] = qq[j] * E[j];
            OpT* QtT_g = reinterpret_cast<OpT*>(ws.QtT) + ch * D * CHUNK;
            store_run<OpT, 8>(QtT_g + frag_off<CHUNK>(cc, r0), qt);
            store_run<OpT, 8>(QtT_g + frag_off<CHUNK>(cc, r0 + 8), qt + 8);
        }
        if (tid < D) ws.gam[ch * D + cc] = egl;
    }

    // CLVR epilogue: the written value v is routed into the hidden stream
    if (hh) {
        const float lm = lam ? lam[h * D + cc] : 1.f;
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            const int r = r0 + j;
            const InT nh = from_f32<InT>(__builtin_fmaf(lm, vv[j], to_f32(hv[j])));
            if constexpr (L::STAGE) HS[r * D + cc] = nh;
            else if (r < nvalid) hh[base + r * tokstride + cc] = nh;
        }
    }
    __syncthreads();  // Kq, Qq (and Kh for scalar gates), block-end values
    if constexpr (L::STAGE) {
        // staged outputs: fragment-order blocks are straight copies; h rows go
        // back to their tokens (rows past the end are not written)
        constexpr int NPC = CHUNK * D * 2 / 16 / NT;  // 16-byte pieces per thread
        if constexpr (QA) {
            uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<OpT*>(ws.Qt) + ch * CHUNK * D);
#pragma unroll
            for (int k2 = 0; k2 < NPC; ++k2) dst[k2 * NT + tid] = reinterpret_cast<const uint4*>(QtS)[k2 * NT + tid];
        }
        if (hh) {
            constexpr int PPR = D * 2 / 16;  // pieces per row
#pragma unroll
            for (int k2 = 0; k2 < NPC; ++k2) {
                const int p = k2 * NT + tid, r = p / PPR, c8 = (p % PPR) * 8;
                if (r < nvalid)
                    *reinterpret_cast<uint4*>(hh + base + r * tokstride + c8) =
                        *reinterpret_cast<const uint4*>(HS + r * D + c8);
            }
        }
    }

    // ---------------- phase 2: P = Kt Kh^T and A = Qt Kh^T on the matrix cores ----------------
    // Tiles are computed transposed (Kh rows as the A operand), so lane l ends up
    // holding P[16R + l%16][16I + 4(l/16) .. +3]: four consecutive columns of one row.
    float* Ps = Nm;  // fp32 P staging, outside the phase 1-2 buffers
    OpT* A_g = reinterpret_cast<OpT*>(ws.A) + ch * CHUNK * CHUNK;
    OpT* AT_g = reinterpret_cast<OpT*>(ws.AT) + ch * CHUNK * CHUNK;
    // One tile job: rows 16R.. of Kq (P) or Qq (A) against the column operand
    // rows kh (16 of them), masked to the lower triangle and stored.
    auto pa_tile = [&](int R, int I, int isA, const OpT* kh) {
        float4v acc = zero4();
        const OpT* arow = kh + l16 * LDR + 8 * g4;
        const OpT* brow = (isA ? Qq : Kq) + (16 * R + l16) * LDR + 8 * g4;
#pragma unroll
        for (int kq = 0; kq < D / 32; ++kq) {
            Frag<OpT> fa, fb;
            fa.load(arow + 32 * kq);
            fb.load(brow + 32 * kq);
            mma(fa, fb, acc);
        }
        const int r = 16 * R + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * g4 + e;
            float f = (i <= r) ? 1.f : 0.f;
            if constexpr (GATE == GATE_SCALAR) f = (i <= r) ? exp2_fast(s_gs[r] - s_gs[i]) : 0.f;
            acc[e] *= f;
        }
        if (isA) {
            if constexpr (QA) store4<OpT>(A_g + frag_off<CHUNK>(r, 16 * I + 4 * g4), acc);
            if constexpr (TR) {
#pragma unroll
                for (int e = 0; e < 4; ++e) AT_g[frag_off<CHUNK>(16 * I + 4 * g4 + e, r)] = from_f32<OpT>(acc[e]);
            }
        } else {
            *reinterpret_cast<float4v*>(Ps + r * CHUNK + 16 * I + 4 * g4) = acc;
        }
    };
    if constexpr (L::KH4) {
        // the column operands of all four block rows (reference ref(R)), built
        // in one pass, so that the 20 tiles need a single barrier
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            if (part <= R) {
                const float ref = R ? s_tot[R - 1][cc] : 0.f;
                const float eref = exp2_fast(ref);
                const bool zero = (part == R) && ((flags >> R) & 1);  // redone exactly below
                OpT* khr = Kh + (8 * R * (R + 1) + r0) * LDR + cc;
#pragma unroll
                for (int j = 0; j < RPP; ++j) {
                    float val = wide ? kk[j] * exp2_fast(ref - G[j]) : kk[j] * (Ei[j] * eref);
                    khr[j * LDR] = from_f32<OpT>(zero ? 0.f : val);
                }
            }
        }
        __syncthreads();
        // tiles (R, I <= R, P or A) in the order R, I, A/P, dealt to the waves in turn
        constexpr int NJOB = 20, JPW = (NJOB + NW - 1) / NW;
#pragma unroll
        for (int k = 0; k < JPW; ++k) {
            const int job = wid + NW * k;
            if (job < NJOB) {
                const int R = job < 2 ? 0 : (job < 6 ? 1 : (job < 12 ? 2 : 3));
                const int I = (job - R * (R + 1)) >> 1, isA = job & 1;
                if (!(I == R && ((flags >> R) & 1))) pa_tile(R, I, isA, Kh + (8 * R * (R + 1) + 16 * I) * LDR);
            }
        }
    } else if constexpr (GATE == GATE_CHANNEL) {
        // fp32 operands: one block row at a time through a single Kh buffer
        int ti = 0;
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            if (part <= R) {
                const float ref = R ? s_tot[R - 1][cc] : 0.f;
                const float eref = exp2_fast(ref);
                const bool zero = (part == R) && ((flags >> R) & 1);  // redone exactly below
#pragma unroll
                for (int j = 0; j < RPP; ++j) {
                    float val = wide ? kk[j] * exp2_fast(ref - G[j]) : kk[j] * (Ei[j] * eref);
                    Kh[(r0 + j) * LDR + cc] = from_f32<OpT>(zero ? 0.f : val);
                }
            }
            __syncthreads();
            for (int I = 0; I <= R; ++I)
                for (int isA = 0; isA < 2; ++isA, ++ti)
                    if ((ti % NW) == wid && !(I == R && ((flags >> R) & 1))) pa_tile(R, I, isA, Kh + (16 * I) * LDR);
            if (R < 3) __syncthreads();  // Kh is rebuilt for the next block row
        }
    } else {
        int ti = 0;
        for (int R = 0; R <= 3; ++R)
            for (int I = 0; I <= R; ++I)
                for (int isA = 0; isA < 2; ++isA, ++ti)
                    if ((ti % NW) == wid) pa_tile(R, I, isA, Kh + (16 * I) * LDR);
    }
    // zero the strictly upper tiles of A (never computed)
    for (int e = tid; e < 6 * 64; e += NT) {
        const int tile = e / 64, w = e % 64;  // tile: (R, I) with I > R
        const int R = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
        const int I = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
        const int r = 16 * R + w / 4, i0 = 16 * I + 4 * (w % 4);
        if constexpr (QA) store4<OpT>(A_g + frag_off<CHUNK>(r, i0), zero4());
        if constexpr (TR) {
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) AT_g[frag_off<CHUNK>(i0 + e2, r)] = from_f32<OpT>(0.f);
        }
    }
    __syncthreads();  // all reads of Kq/Qq/Kh done: the region is reused below

    // Kt^T and V^T operands for W and Ut
    {
        float kt[RPP];
#pragma unroll
        for (int j = 0; j < RPP; ++j) kt[j] = kk[j] * E[j];
        store_run<OpT, RPP>(KtT + cc * LDC + r0, kt);
        store_run<OpT, RPP>(VT + cc * LDC + r0, vv);
    }

    // exact diagonal blocks for the channel gate when the decay range is too wide:
    // 2^(G_r - G_i) = prod_{s=i+1..r} alpha_s, accumulated as a running product
    if constexpr (GATE == GATE_CHANNEL) {
        if (flags && tid < 256) {
            constexpr int CPG = D / 16;  // channels per group
            const int rr = tid >> 4, cg = tid & 15;
#pragma unroll 1
            for (int R = 0; R < 4; ++R) {
                if (!((flags >> R) & 1)) continue;
                const int r = 16 * R + rr;
                const bool okr = r < nvalid;
                float kr[CPG], qr[CPG], f[CPG];
#pragma unroll
                for (int m = 0; m < CPG; ++m) {
                    const int64_t e = base + r * tokstride + cg * CPG + m;
                    kr[m] = okr ? to_f32(k[e]) : 0.f;
                    qr[m] = okr ? to_f32(q[e]) : 0.f;
                    f[m] = 1.f;
                }
#pragma unroll 1
                for (int i = 15; i >= 0; --i) {
                    const int ii = 16 * R + i;
                    float ps = 0.f, as = 0.f;
                    if (ii <= r) {
                        if (ii < r) {  // include alpha_{ii+1}
                            const int s = ii + 1;
                            const bool oks = s < nvalid;
#pragma unroll
                            for (int m = 0; m < CPG; ++m)
                                f[m] *= oks ? alpha[base + s * tokstride + cg * CPG + m] : 1.f;
                        }
                        const bool oki = ii < nvalid;
#pragma unroll
                        for (int m = 0; m < CPG; ++m) {
                            const float ki = oki ? to_f32(k[base + ii * tokstride + cg * CPG + m]) : 0.f;
                            ps += kr[m] * ki * f[m];
                            as += qr[m] * ki * f[m];
                        }
                    }
#pragma unroll
                    for (int off = 1; off < 16; off <<= 1) {
                        ps += __shfl_xor(ps, off);
                        as += __shfl_xor(as, off);
                    }
                    if (cg == 0) {
                        Ps[r * CHUNK + ii] = ps;
                        if constexpr (QA) A_g[frag_off<CHUNK>(r, ii)] = from_f32<OpT>(as);
                        if constexpr (TR) AT_g[frag_off<CHUNK>(ii, r)] = from_f32<OpT>(as);
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---------------- phase 3: T = (I + L)^-1 diag(beta), L = strict_tril(diag(beta) P) ----------------
    // four consecutive elements of one row per thread and step (16-byte accesses)
    for (int e4 = tid; e4 < CHUNK * CHUNK / 4; e4 += NT) {
        const int e = 4 * e4, r = e / CHUNK, i0 = e % CHUNK;
        const float4v pv = *reinterpret_cast<const float4v*>(Ps + e);
        const float br = s_beta[r];
        float4v pw, pm;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pw[c] = (i0 + c < r) ? pv[c] : 0.f;
            pm[c] = (i0 + c < r) ? br * pv[c] : 0.f;
        }
        if constexpr (BWD) *reinterpret_cast<float4v*>(ws.Pw + ch * CHUNK * CHUNK + e) = pw;
        *reinterpret_cast<float4v*>(Pm + e) = pm;
        *reinterpret_cast<float4v*>(Nm + e) = zero4();  // Ps aliases Nm: read above, before the zero
    }
    __syncthreads();
    // diagonal 16x16 blocks, one wave per block, lane j solves column j of
    // (I + L_RR) x = e_j column by column: once x_m is final it is applied to
    // every later row, so the 15 updates of each step are independent
    if (wid < 4 && lane < 16) {
        const int R = wid;
        const float* Lb = Pm + (16 * R) * CHUNK + 16 * R;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == lane) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 15; ++m) {
            const float xm = x[m];
#pragma unroll
            for (int r = m + 1; r < 16; ++r) x[r] -= Lb[r * CHUNK + m] * xm;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Nm[(16 * R + r) * CHUNK + 16 * R + lane] = x[r];
    }
    __syncthreads();
    // off-diagonal blocks, one block row at a time on fp32 matrix cores:
    // N[R, J] = -N_RR (sum_{K=J}^{R-1} L[R, K] N[K, J]), wave J taking tile J.
    // One v_mfma_f32_16x16x4 per 4-wide k slice; lane (l16, g4) supplies k =
    // 4 g4 + m of instruction m, so A rows are read as float4 and the product's
    // accumulator (rows 4 g4 .. +3, column l16) is directly the B operand of
    // the next product.
#pragma unroll
    for (int R = 1; R < 4; ++R) {
        if (wid < R) {
            const int J = wid;
            float4v x = zero4();
            for (int K = J; K < R; ++K) {
                const float4v a = *reinterpret_cast<const float4v*>(Pm + (16 * R + l16) * CHUNK + 16 * K + 4 * g4);
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    x = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], Nm[(16 * K + 4 * g4 + m) * CHUNK + 16 * J + l16], x,
                                                             0, 0, 0);
            }
            const float4v nrr = *reinterpret_cast<const float4v*>(Nm + (16 * R + l16) * CHUNK + 16 * R + 4 * g4);
            float4v y = zero4();
#pragma unroll
            for (int m = 0; m < 4; ++m) y = __builtin_amdgcn_mfma_f32_16x16x4f32(nrr[m], x[m], y, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) Nm[(16 * R + 4 * g4 + e) * CHUNK + 16 * J + l16] = -y[e];
        }
        __syncthreads();
    }
    // T = N diag(beta) in operand precision (row-major, padded), in the L region
    for (int e4 = tid; e4 < CHUNK * CHUNK / 4; e4 += NT) {
        const int e = 4 * e4, r = e / CHUNK, i0 = e % CHUNK;
        const float4v n = *reinterpret_cast<const float4v*>(Nm + e);
        if constexpr (sizeof(OpT) == 2) {
            half4 t;
#pragma unroll
            for (int c = 0; c < 4; ++c) t[c] = from_f32<OpT>(n[c] * s_beta[i0 + c]);
            *reinterpret_cast<half4*>(Tm + r * LDC + i0) = t;
        } else {
            float4v t;
#pragma unroll
            for (int c = 0; c < 4; ++c) t[c] = n[c] * s_beta[i0 + c];
            *reinterpret_cast<float4v*>(Tm + r * LDC + i0) = t;
        }
        if constexpr (BWD) *reinterpret_cast<float4v*>(ws.Nw + ch * CHUNK * CHUNK + e) = n;
    }
    __syncthreads();

    // ---------------- phase 4: W = T Kt and Ut = T V (computed transposed) ----------------
    {
        OpT* W_g = reinterpret_cast<OpT*>(ws.W) + ch * CHUNK * D;
        OpT* U_g = reinterpret_cast<OpT*>(ws.Ut) + ch * CHUNK * D;
        OpT* WT_g = reinterpret_cast<OpT*>(ws.WT) + ch * D * CHUNK;
        for (int m = wid; m < D / 16; m += NW) {
#pragma unroll
            for (int mat = 0; mat < 2; ++mat) {
                const OpT* arow = (mat ? VT : KtT) + (16 * m + l16) * LDC + 8 * g4;
                Frag<OpT> fa0, fa1;
                fa0.load(arow);
                fa1.load(arow + 32);
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    float4v acc = zero4();
                    const OpT* brow = Tm + (16 * n + l16) * LDC + 8 * g4;
                    Frag<OpT> fb;
                    fb.load(brow);
                    mma(fa0, fb, acc);
                    if (n >= 2) {
                        fb.load(brow + 32);
                        mma(fa1, fb, acc);
                    }
                    const int pos = 16 * n + l16, d0 = 16 * m + 4 * g4;
                    if (mat == 0) {
                        store4<OpT>(W_g + frag_off<D>(pos, d0), acc);  // A operand of W S
                        if constexpr (TR) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) WT_g[frag_off<CHUNK>(d0 + e, pos)] = from_f32<OpT>(acc[e]);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) U_g[cfrag_off<D>(pos, d0 + e)] = from_f32<OpT>(acc[e]);
                    }
                }
            }
        }
    }
}

template <int D, int GATE, bool IN_F32>
static hipError_t launch_intra_t(int mode, int64_t B, int64_t T, int H, int64_t NC, const void* q,
                                 const void* k, const void* v, const float* beta,
                                 const float* alpha, void* h_clvr, const float* lam,
                                 const ChunkWs& ws, int pro, ChunkRange cr, hipStream_t stream) {
    const int64_t nblk = B * H * cr.n;
    if (nblk == 0) return hipSuccess;
#define GDR_INTRA(M, P)                                                                                \
    hipLaunchKernelGGL((intra_kernel<D, GATE, IN_F32, M, P>), dim3((unsigned)nblk), dim3(4 * D), 0, stream, T, H, \
                       NC, q, k, v, beta, alpha, h_clvr, lam, ws, pro, cr)
    if (pro) {
        if (mode == 1) GDR_INTRA(1, true);
        else if (mode == 2) GDR_INTRA(2, true);
        else GDR_INTRA(0, true);
    } else {
        if (mode == 1) GDR_INTRA(1, false);
        else if (mode == 2) GDR_INTRA(2, false);
        else GDR_INTRA(0, false);
    }
#undef GDR_INTRA
    return hipGetLastError();
}

template <int D, bool IN_F32>
static hipError_t launch_intra_d(int gate, int mode, int64_t B, int64_t T, int H, int64_t NC,
                                 const void* q, const void* k, const void* v, const float* beta,
                                 const float* alpha, void* h_clvr, const float* lam,
                                 const ChunkWs& ws, int pro, ChunkRange cr, hipStream_t stream) {
    switch (gate) {
        case GATE_NONE: return launch_intra_t<D, GATE_NONE, IN_F32>(mode, B, T, H, NC, q, k, v, beta, alpha, h_clvr, lam, ws, pro, cr, stream);
        case GATE_SCALAR: return launch_intra_t<D, GATE_SCALAR, IN_F32>(mode, B, T, H, NC, q, k, v, beta, alpha, h_clvr, lam, ws, pro, cr, stream);
        default: return launch_intra_t<D, GATE_CHANNEL, IN_F32>(mode, B, T, H, NC, q, k, v, beta, alpha, h_clvr, lam, ws, pro, cr, stream);
    }
}

hipError_t launch_intra(int D, int gate, bool in_f32, int mode, int64_t B, int64_t T, int H,
                        int64_t NC, const void* q, const void* k, const void* v,
                        const float* beta, const float* alpha, void* h_clvr, const float* lam,
                        const ChunkWs& ws, int pro, ChunkRange cr, hipStream_t stream) {
    if (D == 64) {
        if (in_f32) return launch_intra_d<64, true>(gate, mode, B, T, H, NC, q, k, v, beta, alpha, h_clvr, lam, ws, pro, cr, stream);
        return launch_intra_d<64, false>(gate, mode, B, T, H, NC, q, k, v, beta, alpha, h_clvr, lam, ws, pro, cr, stream);
    }
    if (in_f32) return launch_intra_d<128, true>(gate, mode, B, T, H, NC, q, k, v, beta, alpha, h_clvr, lam, ws, pro, cr, stream);
    return launch_intra_d<128, false>(gate, mode, B, T, H, NC, q, k, v, beta, alpha, h_clvr, lam, ws, pro, cr, stream);
}

}  // namespace gdr
