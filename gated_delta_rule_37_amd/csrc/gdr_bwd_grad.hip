// gdr_bwd_grad.hip -- per-chunk gradients of the chunked gated delta rule.
//
// With S the chunk-start state, dS' the chunk-end state gradient and dU, U, dO
// (scaled by the output scale) of the chunk, the chunk's forward
//   U = T (V - Kt S),  O = Qt S + A U,  S' = Diag(gamma) S + Kb^T U,
//   T = N diag(beta),  N = (I + L)^-1,  L = strict_tril(diag(beta) P),
//   P = Kt Kh^T,  A = tril(Qt Kh^T),  W = T Kt, Ut = T V
// gives, in reverse mode (every identity below is the derivative of one line):
//   dQt = dO S^T               dA = tril(dO U^T)        dKb = U dS'^T
//   dW  = -dU S^T              dgamma = rowsum(dS' . S)
//   dT  = dU V^T + dW Kt^T     dV = T^T dU              dKt = T^T dW
//   Y   = N^T dT               dbeta = diag(Y) + rowsum(dL . P)
//   dL  = -strict_tril(Y T^T)  dP = diag(beta) dL
// The first stage (grad_lin_body) computes all of that.  The second
// (grad_gate_body) takes dA and dP back through the decay-factored products
// (the same block references as the forward), adds the Qt, Kt, Kb and gamma
// terms, and turns the gradient with respect to the in-chunk log-decay cumsum
// into dalpha by a reverse cumsum.  One workgroup runs both for a chunk.
#include "gdr_cler.hpp"
#include "gdr_common.hpp"
#include "gdr_launch.hpp"

#include <type_traits>

namespace gdr {

// NORO: the row operands dO, dU and U are read from global memory where they
// are used instead of being staged in LDS (fp32 operands at d = 128, where the
// staging does not fit).
template <int D, bool IN_F32, bool NORO = false>
struct GLinLayout {
    using OpT = typename std::conditional<IN_F32, float, _Float16>::type;
    static constexpr int OPB = sizeof(OpT);
    static constexpr int PAD = 16 / OPB;
    static constexpr int LDR = D + PAD;
    static constexpr int LDC = CHUNK + PAD;
    static constexpr int NT = 4 * D;
    static constexpr int NW = NT / WAVE;
    static constexpr int KT = 0;                           // Kt [64][LDR]  (Kt and dW later: Y fp32)
    static constexpr int DW = KT + CHUNK * LDR * OPB;      // dW [64][LDR]
    static constexpr int DWT = DW + CHUNK * LDR * OPB;     // dW^T [D][LDC]
    static constexpr int TT = DWT + D * LDC * OPB;         // T^T [64][LDC]
    static constexpr int LDF = CHUNK + 4;                  // fp32 row stride (16-byte pad)
    static constexpr int NF = TT + CHUNK * LDC * OPB;      // N [64][LDF] fp32
    static constexpr int DTF = NF + CHUNK * LDF * 4;       // dT [64][LDF] fp32, later Y
    static constexpr int RO = DTF + CHUNK * LDF * 4;       // row operands of phase 1, fragment order:
    static constexpr int RDO = RO;                         //   scaled-free dO [64][D]
    static constexpr int RDU = RDO + CHUNK * D * OPB;      //   dU [64][D]
    static constexpr int RU = RDU + CHUNK * D * OPB;       //   U [64][D]
    static constexpr int BYTES = NORO ? RO : RU + CHUNK * D * OPB;
    // phase 3 reuses the Kt..T^T region (dead by then) for N^T and dT^T (fp32)
    static_assert(2 * CHUNK * LDF * 4 <= NF, "N^T and dT^T must fit below N");
};

// LDS layout of the second stage (defined here: the first stage writes into it).
template <int D, bool IN_F32>
struct GGateLayout {
    using OpT = typename std::conditional<IN_F32, float, _Float16>::type;
    static constexpr int OPB = sizeof(OpT);
    static constexpr int PAD = 16 / OPB;
    static constexpr int LDC = CHUNK + PAD;
    static constexpr int NT = 4 * D;
    static constexpr int NW = NT / WAVE;
    static constexpr int DA = 0;                            // dA  [64][LDC]
    static constexpr int DP = DA + CHUNK * LDC * OPB;       // dP  [64][LDC]
    static constexpr int DAT = DP + CHUNK * LDC * OPB;      // dA^T
    static constexpr int DPT = DAT + CHUNK * LDC * OPB;     // dP^T
    static constexpr int QQT = DPT + CHUNK * LDC * OPB;     // Qq^T [D][LDC]
    static constexpr int KQT = QQT + D * LDC * OPB;         // Kq^T
    static constexpr int KHT = KQT + D * LDC * OPB;         // Kh^T
    static constexpr int SA = KHT + D * LDC * OPB;          // fp32 [16][D]  dA_R Kh
    static constexpr int SB = SA + 16 * D * 4;              // fp32 [16][D]  dP_R Kh
    static constexpr int SC = SB + 16 * D * 4;              // fp32 [64][D]  dA_R^T Qq + dP_R^T Kq
    static constexpr int BYTES = SC + CHUNK * D * 4;
    static constexpr float RHO_MAX = IN_F32 ? 100.f : 8.f;
    // on-chip partials: dQt, dKt, dKb handed to the combine through LDS that is
    // free by then (SA .. the end, else dA .. dP^T), [D][64] each with the
    // 16-byte pieces of a column XOR-swizzled by the column
    static constexpr int XPART = 3 * CHUNK * D * OPB;
    static constexpr int XR = (BYTES - SA >= XPART) ? SA : DA;
    static_assert(XR == SA || QQT - DA >= XPART, "partials exchange fits");
    static constexpr int EPC = 16 / OPB;       // elements per 16-byte piece
    static constexpr int NPC = CHUNK / EPC;    // pieces per column
};

// Offset of (row r, column c) in one [D][64] array of the partials exchange.
template <int EPC, int NPC>
__device__ __forceinline__ int xoff(int c, int r) {
    return c * CHUNK + (((r / EPC) ^ (c % NPC)) * EPC) + r % EPC;
}

// The first stage's partials (dQt, dKb, dKt, dA, dP) as the second stage takes
// them when they stay on chip: this thread's values in the accumulator layout
// they were computed in (four consecutive rows of one column per tile), in
// operand precision, so they are rounded exactly as the workspace copies are.
template <int D, bool IN_F32>
struct GradPartials {
    using V4 = typename std::conditional<IN_F32, float4v, half4>::type;
    static constexpr int NW = 4 * D / WAVE;
    static constexpr int NHALF = NW / 4;
    static constexpr int NIT = D / 16 / NHALF;  // dKt column tiles per wave
    static constexpr int NPW = 4 / NHALF;       // dA position tiles per wave
    static constexpr int NTL = 16 / NW;         // dP tiles per wave
    // Where each stays: at d = 64 (one wave per SIMD, registers to spare) all in
    // registers; at d = 128 dKt goes to LDS past the second stage's buffers and
    // dQt, dKb still through the workspace (holding them too would spill).
    static constexpr bool QREG = grad_qkb_on_chip(D);
    static constexpr bool TLDS = D == 128;
    V4 q[4], kb[4];  // dQt, dKb: row tile r4, value-column tile = wave
    V4 kt[NIT];      // dKt: row tile wave % 4, value-column tiles wave / 4 + NHALF i
    V4 a[NPW];       // dA: row tiles wave / 4 + NHALF k, column tile wave % 4
    V4 p[NTL];       // dP: tile wave + NW t
};

template <typename V4>
__device__ __forceinline__ V4 to_v4(const float (&x)[4]) {
    V4 r;
    using E = typename std::remove_reference<decltype(r[0])>::type;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = from_f32<E>(x[e]);
    return r;
}

template <typename InT, typename OpT>
__device__ __forceinline__ void load_frag_in(Frag<OpT>& f, const InT* p) {
    // eight consecutive input elements -> operand precision
    if constexpr (sizeof(InT) == 2) {
        const uint4 raw = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f.v[2 * e] = static_cast<OpT>(__uint_as_float(w[e] << 16));
            f.v[2 * e + 1] = static_cast<OpT>(__uint_as_float(w[e] & 0xffff0000u));
        }
    } else {
        const float4v a = reinterpret_cast<const float4v*>(p)[0];
        const float4v b = reinterpret_cast<const float4v*>(p)[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f.v[e] = static_cast<OpT>(a[e]);
            f.v[4 + e] = static_cast<OpT>(b[e]);
        }
    }
}

// The two gradient stages are device functions on a caller-provided LDS
// buffer, which grads_kernel runs one after the other for a chunk.
// KEEP: the partials stay on chip (pk, and dgamma in s_gam) instead of going
// through the workspace.
// ROUTE only tells the value route's and the error route's instances apart.
template <int D, int GATE, bool IN_F32, bool OUT_F32, bool PRO, bool KEEP, bool NORO = false, int ROUTE = 0>
__device__ __forceinline__ void grad_lin_body(int64_t T, int H, int64_t NC, float scale,
                                              const void* __restrict__ k_, const void* __restrict__ v_,
                                              const float* __restrict__ beta, const float* __restrict__ alpha,
                                              const void* __restrict__ dO_, const void* __restrict__ dh_,
                                              const float* __restrict__ lam, void* __restrict__ dv_,
                                              float* __restrict__ dbeta, ChunkWs ws, int pro,
                                              ChunkRange cr, char* smem, GradPartials<D, IN_F32>& pk,
                                              float* s_gam, float (&s_tot)[4][D]) {
    using L = GLinLayout<D, IN_F32, NORO>;
    using OpT = typename L::OpT;
    using InT = typename InType<IN_F32>::T;
    using OutT = typename InType<OUT_F32>::T;
    constexpr int NT = L::NT, NW = L::NW, LDR = L::LDR, LDC = L::LDC, LDF = L::LDF, RPP = 16;

    __shared__ float s_gs[CHUNK];
    __shared__ float s_beta[CHUNK];
    __shared__ float s_db[CHUNK];
    __shared__ float s_rk[PRO ? CHUNK : 1];  // prologue: reciprocal k row norms

    OpT* KT = reinterpret_cast<OpT*>(smem + L::KT);
    float* NTF = reinterpret_cast<float*>(smem + L::KT);                    // phase 3: N^T
    float* DTT = reinterpret_cast<float*>(smem + L::KT + CHUNK * LDF * 4);  // phase 3: dT^T
    OpT* DWs = reinterpret_cast<OpT*>(smem + L::DW);
    OpT* DWT = reinterpret_cast<OpT*>(smem + L::DWT);
    OpT* TT = reinterpret_cast<OpT*>(smem + L::TT);
    float* NF = reinterpret_cast<float*>(smem + L::NF);
    float* DTF = reinterpret_cast<float*>(smem + L::DTF);

    int64_t bh, c;
    range_block(cr, bh, c);
    const int64_t ch = bh * NC + c;
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh % H);
    const int64_t t0 = c * CHUNK;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int cc = tid % D, part = tid / D, r0 = part * RPP;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t tokstride = static_cast<int64_t>(H) * D;
    const int64_t base = ((b * T + t0) * H + h) * D;
    const int64_t nvalid64 = T - t0;
    const int nvalid = nvalid64 < CHUNK ? static_cast<int>(nvalid64) : CHUNK;
    const InT* k = reinterpret_cast<const InT*>(k_);
    const InT* v = reinterpret_cast<const InT*>(v_);
    const InT* dO = reinterpret_cast<const InT*>(dO_);

    // ---------------- loads.  Phase 0's operands (beta, alpha, k, N) are issued
    // first, so that phase 0 waits only for them; phase 1's (dU and U copied to
    // LDS, dO, and this wave's S, dS' and V fragments) follow and land while
    // phase 0 computes.
    float bt0 = 0.f, rk0 = 0.f, at0 = 1.f;
    const bool tok_ok = tid < nvalid;
    if (tid < CHUNK) {
        const int64_t tok = (b * T + t0 + (tok_ok ? tid : nvalid - 1)) * H + h;
        bt0 = beta[tok];  // activated (the prologue's copy when it is on)
        if constexpr (PRO) rk0 = ws.rk[tok];
        if constexpr (GATE == GATE_SCALAR) at0 = alpha[tok];
    }
    float G[RPP], kk[RPP];
#pragma unroll
    for (int j = 0; j < RPP; ++j) {
        const int r = r0 + j;
        const int64_t e = base + (r < nvalid ? r : nvalid - 1) * tokstride + cc;
        kk[j] = to_f32(k[e]);
        if constexpr (GATE == GATE_CHANNEL) G[j] = alpha[e];
        else G[j] = 0.f;
    }
    constexpr int NE = CHUNK * CHUNK / NT;
    float nv[NE];
#pragma unroll
    for (int k2 = 0; k2 < NE; ++k2) nv[k2] = ws.Nw[ch * CHUNK * CHUNK + k2 * NT + tid];

    constexpr int KQ1 = D / 32;
    OpT* sDO = reinterpret_cast<OpT*>(smem + L::RDO);
    const OpT* Ss = reinterpret_cast<const OpT*>(ws.Ssnap) + ch * D * D;
    const OpT* dSs = reinterpret_cast<const OpT*>(ws.dSsnap) + ch * D * D;
    Frag<OpT> bS[KQ1], bV[KQ1];
    Frag<OpT> bD[KQ1];
    const int itp = wid & 3;
    constexpr int NP = CHUNK * D / 8 / NT;  // dO: 8-element pieces per thread
    Frag<OpT> xdo[NP];
    constexpr int NCPT = CHUNK * D * L::OPB / 16 / NT;  // dU, U: 16-byte pieces per thread
    uint4v xdu[NCPT], xu[NCPT];
    {
        constexpr int KQ = KQ1;
        // dU and U: 16-byte pieces into registers, written to LDS at the start of
        // phase 1.  (Not direct-to-LDS copies: while one of those is pending the
        // compiler makes every LDS access wait for all loads, phase 0's included.)
        if constexpr (!NORO) {
            const uint4v* gdu = reinterpret_cast<const uint4v*>(static_cast<const char*>(ws.dUsave) + ch * CHUNK * D * L::OPB);
            const uint4v* gu = reinterpret_cast<const uint4v*>(static_cast<const char*>(ws.Usave) + ch * CHUNK * D * L::OPB);
#pragma unroll
            for (int it = 0; it < NCPT; ++it) {
                xdu[it] = gdu[it * NT + tid];
                xu[it] = gu[it * NT + tid];
            }
        }
        // this wave's column tile of S and dS' (B operands, k = value column)
        const int nt = wid;
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq) {
            bS[kq].load(Ss + ((nt * KQ + kq) * 64 + lane) * 8);
            bD[kq].load(dSs + ((nt * KQ + kq) * 64 + lane) * 8);
        }
        // V rows of this wave's position tiles (it = wid % 4); rows past the end
        // read the last row and are zeroed at use
        {
            const int brow = 16 * itp + l16;
            const int64_t brow_g = base + (brow < nvalid ? brow : nvalid - 1) * tokstride;
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq) load_frag_in<InT, OpT>(bV[kq], v + brow_g + 32 * kq + 8 * g4);
        }
        // dO pieces, converted into LDS at the start of phase 1
        if constexpr (!NORO) {
#pragma unroll
            for (int k2 = 0; k2 < NP; ++k2) {
                const int p = k2 * NT + tid, f = p >> 6, l = p & 63;
                const int pos = 16 * (f / KQ) + (l & 15), j = 32 * (f % KQ) + 8 * (l >> 4);
                load_frag_in<InT, OpT>(xdo[k2], dO + base + (pos < nvalid ? pos : nvalid - 1) * tokstride + j);
            }
        }
    }

    // ---------------- phase 0: Kt = K 2^G, N, T^T ----------------
    if (tid < CHUNK) {
        s_beta[tid] = tok_ok ? bt0 : 0.f;
        if constexpr (PRO) s_rk[tid] = rk0;  // prologue: k row norms (intra kernel; negative if clamped)
        if constexpr (GATE == GATE_SCALAR) {
            float g = tok_ok ? (PRO ? log2_alpha_logit(at0, pro) : log2_fast(at0)) : 0.f;
            s_gs[tid] = chunk_prefix_sum(g);
        }
    }
#pragma unroll
    for (int j = 0; j < RPP; ++j) {
        const bool ok = r0 + j < nvalid;
        kk[j] = ok ? kk[j] : 0.f;
        if constexpr (GATE == GATE_CHANNEL) G[j] = ok ? (PRO ? log2_alpha_logit(G[j], pro) : log2_fast(G[j])) : 0.f;
    }
    if constexpr (GATE == GATE_CHANNEL) {
#pragma unroll
        for (int j = 1; j < RPP; ++j) G[j] += G[j - 1];
        s_tot[part][cc] = G[RPP - 1];
    }
#pragma unroll
    for (int k2 = 0; k2 < NE; ++k2) {
        const int e = k2 * NT + tid;
        NF[(e / CHUNK) * LDF + e % CHUNK] = nv[k2];
    }
    __syncthreads();
    if constexpr (GATE == GATE_CHANNEL) {
        float carry = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p) carry += (p < part) ? s_tot[p][cc] : 0.f;
#pragma unroll
        for (int j = 0; j < RPP; ++j) G[j] += carry;
    } else if constexpr (GATE == GATE_SCALAR) {
#pragma unroll
        for (int j = 0; j < RPP; ++j) G[j] = s_gs[r0 + j];
    }
#pragma unroll
    for (int j = 0; j < RPP; ++j) {
        // prologue: k divided by its row norm
        const float kn = PRO ? kk[j] * fabsf(s_rk[r0 + j]) : kk[j];
        KT[(r0 + j) * LDR + cc] = from_f32<OpT>(kn * exp2_fast(G[j]));
    }
    // T^T[i][r] = N[r][i] beta_i
    for (int e = tid; e < CHUNK * CHUNK; e += NT) {
        const int r = e / CHUNK, i = e % CHUNK;
        TT[i * LDC + r] = from_f32<OpT>(NF[r * LDF + i] * s_beta[i]);
    }
    __syncthreads();

    // ---------------- phase 1: products contracting over the value dimension ----------------
    // The row operands (dO, dU, U; 16 rows per tile) are staged in LDS once.
    // Wave w owns value-column tile w (D/16 tiles, one per wave) of dQt = dO S^T,
    // dW = -dU S^T and dKb = U dS'^T for all four row tiles, so S and dS' are
    // read from global memory exactly once; dgamma comes from the same
    // registers.  The position tiles (dA, dT1) are spread four per column of
    // waves.  Global stores wait until every load of the phase is issued.
    constexpr int NHALF = NW / 4;
    const int rt = wid & 3, half = wid >> 2;
    {
        constexpr int KQ = D / 32;
        const OpT* sDU = reinterpret_cast<const OpT*>(smem + L::RDU);
        const OpT* sU = reinterpret_cast<const OpT*>(smem + L::RU);
        constexpr int NPW = 4 / NHALF;  // position tiles per wave
        const int nt = wid;             // this wave's value-column tile
        // dU and U into LDS; dO converted (rows past the end zero); V rows past
        // the end zeroed
        if constexpr (!NORO) {
            uint4v* sdu = reinterpret_cast<uint4v*>(smem + L::RDU);
            uint4v* su = reinterpret_cast<uint4v*>(smem + L::RU);
#pragma unroll
            for (int it = 0; it < NCPT; ++it) {
                sdu[it * NT + tid] = xdu[it];
                su[it * NT + tid] = xu[it];
            }
        }
#pragma unroll
        for (int k2 = 0; k2 < (NORO ? 0 : NP); ++k2) {
            const int p = k2 * NT + tid, f = p >> 6, l = p & 63;
            if (16 * (f / KQ) + (l & 15) >= nvalid) xdo[k2].zero();
            if constexpr (sizeof(OpT) == 2) {
                *reinterpret_cast<half8*>(sDO + p * 8) = xdo[k2].v;
            } else {
                float4v lo, hi;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo[e] = xdo[k2].v[e];
                    hi[e] = xdo[k2].v[4 + e];
                }
                reinterpret_cast<float4v*>(sDO + p * 8)[0] = lo;
                reinterpret_cast<float4v*>(sDO + p * 8)[1] = hi;
            }
        }
        if (16 * itp + l16 >= nvalid) {
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq) bV[kq].zero();
        }
        __syncthreads();

        // dgamma_d = sum_j dS'[d][j] S[d][j], d = 16 nt + l16: this lane's 8 KQ
        // columns, then the four lane groups in a fixed order
        float sg = 0.f;
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq)
#pragma unroll
            for (int e = 0; e < 8; ++e) sg += static_cast<float>(bS[kq].v[e]) * static_cast<float>(bD[kq].v[e]);
        sg += __shfl_xor(sg, 16);
        sg += __shfl_xor(sg, 32);

        // fragment (row tile r4, 32-column step kq) of dO, dU or U
        const OpT* gDU = reinterpret_cast<const OpT*>(ws.dUsave) + ch * CHUNK * D;
        const OpT* gU = reinterpret_cast<const OpT*>(ws.Usave) + ch * CHUNK * D;
        auto ld_do = [&](Frag<OpT>& f, int r4, int kq) {
            if constexpr (NORO) {
                const int pos = 16 * r4 + l16;
                load_frag_in<InT, OpT>(f, dO + base + (pos < nvalid ? pos : nvalid - 1) * tokstride + 32 * kq + 8 * g4);
                if (pos >= nvalid) f.zero();
            } else {
                f.load(sDO + ((r4 * KQ + kq) * 64 + lane) * 8);
            }
        };
        auto ld_du = [&](Frag<OpT>& f, int r4, int kq) {
            f.load((NORO ? gDU : sDU) + ((r4 * KQ + kq) * 64 + lane) * 8);
        };
        auto ld_u = [&](Frag<OpT>& f, int r4, int kq) {
            f.load((NORO ? gU : sU) + ((r4 * KQ + kq) * 64 + lane) * 8);
        };
        float rq[4][4], rk[4][4], ra[NPW][4];
        const int col = 16 * nt + l16;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            float4v aq = zero4(), aw = zero4(), ak = zero4();
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq) {
                Frag<OpT> fo_, fdu, fu;
                ld_do(fo_, r4, kq);
                ld_du(fdu, r4, kq);
                ld_u(fu, r4, kq);
                mma(fo_, bS[kq], aq);
                mma(fdu, bS[kq], aw);
                mma(fu, bD[kq], ak);
            }
            const int r0_ = 16 * r4 + 4 * g4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                rq[r4][e] = scale * aq[e];
                rk[r4][e] = ak[e];
                const OpT w = from_f32<OpT>(-aw[e]);
                DWs[(r0_ + e) * LDR + col] = w;
                DWT[col * LDC + r0_ + e] = w;
            }
        }
        // position tiles: dA = tril(dO U^T) (scaled), dT1 = dU V^T
        Frag<OpT> bU[KQ];
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq) ld_u(bU[kq], itp, kq);
#pragma unroll
        for (int k = 0; k < NPW; ++k) {
            const int r4 = (wid >> 2) + k * NHALF;
            float4v aa = zero4(), at = zero4();
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq) {
                Frag<OpT> fo_, fdu;
                ld_do(fo_, r4, kq);
                ld_du(fdu, r4, kq);
                mma(fo_, bU[kq], aa);  // tiles above the diagonal are masked below (no branch here)
                mma(fdu, bV[kq], at);
            }
            const int r0_ = 16 * r4 + 4 * g4, pc = 16 * itp + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ra[k][e] = (pc <= r0_ + e) ? scale * aa[e] : 0.f;
                DTF[(r0_ + e) * LDF + pc] = at[e];
            }
        }
        // stores (or the on-chip copies)
        using P = GradPartials<D, IN_F32>;
        if constexpr (KEEP) {
            using V4 = typename P::V4;
            if constexpr (P::QREG) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    pk.q[r4] = to_v4<V4>(rq[r4]);
                    pk.kb[r4] = to_v4<V4>(rk[r4]);
                }
            }
#pragma unroll
            for (int k = 0; k < NPW; ++k) pk.a[k] = to_v4<V4>(ra[k]);
            if (g4 == 0) s_gam[col] = sg;
        }
        if constexpr (!KEEP || !P::QREG) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    static_cast<OpT*>(ws.gQt)[ch * CHUNK * D + (16 * r4 + 4 * g4 + e) * D + col] =
                        from_f32<OpT>(rq[r4][e]);
                    static_cast<OpT*>(ws.gKb)[ch * CHUNK * D + (16 * r4 + 4 * g4 + e) * D + col] =
                        from_f32<OpT>(rk[r4][e]);
                }
            }
        }
        if constexpr (!KEEP) {
#pragma unroll
            for (int k = 0; k < NPW; ++k) {
                const int r4 = (wid >> 2) + k * NHALF;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    static_cast<OpT*>(ws.gA)[ch * CHUNK * CHUNK + (16 * r4 + 4 * g4 + e) * CHUNK + 16 * itp + l16] =
                        from_f32<OpT>(ra[k][e]);
            }
            if (g4 == 0) ws.gGam[ch * D + col] = sg;
        }
    }
    __syncthreads();

    // ---------------- phase 2: dT += dW Kt^T, dKt = T^T dW, dV = T^T dU ----------------
    {
        OutT* dv = reinterpret_cast<OutT*>(dv_);
        const InT* dh = reinterpret_cast<const InT*>(dh_);
        const int r_ = 16 * rt + 4 * g4;
        Frag<OpT> aT[2];
        aT[0].load(TT + (16 * rt + l16) * LDC + 8 * g4);
        aT[1].load(TT + (16 * rt + l16) * LDC + 32 + 8 * g4);
        // global loads first (the CLVR terms, fp32: dU^T fragments), stores last.
        // fp16: dU^T's fragments (k = position, n = value column) are column
        // pieces of dU's fragment-order LDS copy, read with transposed reads
        constexpr int NIT = D / 16 / NHALF;
        Frag<OpT> bU[NIT][2];
        float dhv[NIT][4], lmv[NIT];
        if constexpr (sizeof(OpT) == 2 && !NORO) {
            const OpT* sDU = reinterpret_cast<const OpT*>(smem + L::RDU);
#pragma unroll
            for (int ct = half; ct < D / 16; ct += NHALF) {
                const int ii = (ct - half) / NHALF;
#pragma unroll
                for (int kq = 0; kq < 2; ++kq) {
                    OpT x[8];
                    lds_column8_at(sDU, 32 * kq + 8 * g4, 16 * ct, lane, [](int r, int c) { return frag_off<D>(r, c); },
                                   x);
#pragma unroll
                    for (int e = 0; e < 8; ++e) bU[ii][kq].v[e] = x[e];
                }
            }
        } else {
            const OpT* dUT = reinterpret_cast<const OpT*>(ws.dUsaveT) + ch * D * CHUNK;
#pragma unroll
            for (int ct = half; ct < D / 16; ct += NHALF) {
                const int ii = (ct - half) / NHALF;
#pragma unroll
                for (int kq = 0; kq < 2; ++kq) bU[ii][kq].load(dUT + ((ct * 2 + kq) * 64 + lane) * 8);
            }
        }
        if (dh) {  // CLVR: the four dh rows of each tile, all issued before any is used
#pragma unroll
            for (int ct = half; ct < D / 16; ct += NHALF) {
                const int ii = (ct - half) / NHALF, col = 16 * ct + l16;
                lmv[ii] = lam ? lam[h * D + col] : 1.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = r_ + e < nvalid ? r_ + e : nvalid - 1;  // clamped; not stored past the end
                    dhv[ii][e] = to_f32(dh[base + r * tokstride + col]);
                }
            }
        } else {
#pragma unroll
            for (int ii = 0; ii < NIT; ++ii) {
                lmv[ii] = 1.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) dhv[ii][e] = 0.f;
            }
        }
        float rkt[NIT][4], rdv[NIT][4];
#pragma unroll
        for (int ct = half; ct < D / 16; ct += NHALF) {
            const int ii = (ct - half) / NHALF;
            Frag<OpT> bW[2];
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) bW[kq].load(DWT + (16 * ct + l16) * LDC + 32 * kq + 8 * g4);
            float4v ak = zero4(), av = zero4();
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                mma(aT[kq], bW[kq], ak);
                mma(aT[kq], bU[ii][kq], av);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                rkt[ii][e] = ak[e];
                rdv[ii][e] = dh ? __builtin_fmaf(lmv[ii], dhv[ii][e], av[e]) : av[e];  // CLVR: h += lam v
            }
        }
#pragma unroll
        for (int ct = half; ct < D / 16; ct += NHALF) {
            const int ii = (ct - half) / NHALF, col = 16 * ct + l16;
            using P = GradPartials<D, IN_F32>;
            if constexpr (KEEP && P::TLDS) {
                // past the second stage's buffers, in its exchange layout (that
                // region lies in the row-operand staging, dead since phase 1)
                using GL = GGateLayout<D, IN_F32>;
                *reinterpret_cast<typename P::V4*>(reinterpret_cast<OpT*>(smem + GL::BYTES) +
                                                   xoff<GL::EPC, GL::NPC>(col, r_)) =
                    to_v4<typename P::V4>(rkt[ii]);
            } else if constexpr (KEEP) {
                pk.kt[ii] = to_v4<typename P::V4>(rkt[ii]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (!KEEP)
                    static_cast<OpT*>(ws.gKt)[ch * CHUNK * D + (r_ + e) * D + col] = from_f32<OpT>(rkt[ii][e]);
                const int r = r_ + e;
                if (r < nvalid) dv[base + r * tokstride + col] = from_f32<OutT>(rdv[ii][e]);
            }
        }
#pragma unroll
        for (int it = half; it < 4; it += NHALF) {
            float4v acc = zero4();
#pragma unroll
            for (int kq = 0; kq < D / 32; ++kq) {
                Frag<OpT> fa, fb;
                fa.load(DWs + (16 * rt + l16) * LDR + 32 * kq + 8 * g4);
                fb.load(KT + (16 * it + l16) * LDR + 32 * kq + 8 * g4);
                mma(fa, fb, acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) DTF[(r_ + e) * LDF + 16 * it + l16] += acc[e];
        }
    }
    __syncthreads();

    // ---------------- phase 3: solve adjoint on fp32 matrix cores ----------------
    // Y = N^T dT and dL = -strict_tril(Y T^T), T = N diag(beta)
    // this wave's P entries of its dL tiles, fetched now so the loads overlap Y
    constexpr int NTL = 16 / NW;
    float pwv[NTL][4];
    {
        const float* Pw = ws.Pw + ch * CHUNK * CHUNK;
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            const int tile = wid + t * NW, at = tile / 4, xt = tile % 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) pwv[t][e] = Pw[(16 * at + 4 * g4 + e) * CHUNK + 16 * xt + l16];
        }
    }
    for (int e = tid; e < CHUNK * CHUNK; e += NT) {
        const int r = e / CHUNK, x = e % CHUNK;
        NTF[x * LDF + r] = NF[r * LDF + x];
        DTT[x * LDF + r] = DTF[r * LDF + x];
    }
    __syncthreads();
    for (int tile = wid; tile < 16; tile += NW) {  // Y tile (at, xt), k = r
        const int at = tile / 4, xt = tile % 4;
        float4v acc = zero4();
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
            Frag<float> fa, fb;
            fa.load(NTF + (16 * at + l16) * LDF + 32 * kq + 8 * g4);
            fb.load(DTT + (16 * xt + l16) * LDF + 32 * kq + 8 * g4);
            mma(fa, fb, acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) DTF[(16 * at + 4 * g4 + e) * LDF + 16 * xt + l16] = acc[e];  // Y
    }
    __syncthreads();
    float* YF = DTF;
    float* CB = NTF;  // dL . P contributions [64][LDF] (N^T is no longer needed)
    {
#pragma unroll
        for (int t = 0; t < NTL; ++t) {  // dL tile (at, xt), k = c
            const int tile = wid + t * NW, at = tile / 4, xt = tile % 4;
            float4v acc = zero4();
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                Frag<float> fa, fb;
                fa.load(YF + (16 * at + l16) * LDF + 32 * kq + 8 * g4);
                const int c0 = 32 * kq + 8 * g4;
                fb.load(NF + (16 * xt + l16) * LDF + c0);  // T[x][c] = N[x][c] beta_c
#pragma unroll
                for (int e = 0; e < 8; ++e) fb.v[e] *= s_beta[c0 + e];
                mma(fa, fb, acc);
            }
            const int x = 16 * xt + l16;
            float dpv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int a = 16 * at + 4 * g4 + e;
                const float dl = (x < a) ? -acc[e] : 0.f;
                dpv[e] = s_beta[a] * dl;
                if constexpr (!KEEP)
                    static_cast<OpT*>(ws.gP)[ch * CHUNK * CHUNK + a * CHUNK + x] = from_f32<OpT>(dpv[e]);
                CB[a * LDF + x] = dl * pwv[t][e];
            }
            if constexpr (KEEP) pk.p[t] = to_v4<typename GradPartials<D, IN_F32>::V4>(dpv);
        }
    }
    __syncthreads();
    if (tid < CHUNK) {  // fixed-order row sums: deterministic
        float sdb = YF[tid * LDF + tid];
        for (int x = 0; x < CHUNK; ++x) sdb += CB[tid * LDF + x];
        s_db[tid] = sdb;
    }
    __syncthreads();
    if (tid < nvalid) {
        float db = s_db[tid];
        if constexpr (PRO) db *= s_beta[tid] * (1.f - s_beta[tid]);  // prologue: beta = sigmoid(logit)
        dbeta[(b * T + t0 + tid) * H + h] = db;
    }
}


}  // namespace gdr

namespace gdr {

// ---------------------------------------------------------------------------
// grad_gate: dA and dP back through the decay-factored products.
//
// With E_ri = 2^(G_r - G_i) (r >= i), A_ri = sum_c q_rc k_ic E_ric and
// P_ri = sum_c k_rc k_ic E_ric.  For block row R and its reference ref(R)
// (G at the last row before the block), Fq_r = 2^(G_r - ref) <= 1 and
// Fh_i = 2^(ref - G_i), so that
//   row side:    dqA_r  = Fq_r . (dA_R Kh)_r      dkP_r  = Fq_r . (dP_R Kh)_r
//   column side: dkC_i += Fh_i . (dA_R^T Qq_R + dP_R^T Kq_R)_i
// with Kh = K . Fh, Qq = Q . Fq, Kq = K . Fq.  The log-decay gradient is then
// elementwise: dG_r += q_r . dqA_r + k_r . dkP_r - k_r . dkC_r.  Adding the Qt,
// Kt, Kb and gamma terms (Qt = Q 2^G, Kt = K 2^G, Kb = K 2^(G_last - G),
// gamma = 2^G_last) gives dq, dk and dG; dalpha_s = (sum_{r >= s} dG_r) / alpha_s
// (G is the cumsum of log alpha).  Diagonal blocks whose decay range is too wide
// for the operand precision are done exactly in fp32 by the thread that owns
// the block's rows (pair factors from G differences, always <= 1).
// ---------------------------------------------------------------------------

// N values of one thread in operand precision, read one by one; fp16 values
// are kept two to a register (the loads fill the low and high halves).
template <typename OpT, int N>
struct PairRows {
    OpT v[N];
    __device__ __forceinline__ void set(int j, OpT x) { v[j] = x; }
    __device__ __forceinline__ float operator[](int j) const { return to_f32(v[j]); }
};
template <int N>
struct PairRows<_Float16, N> {
    typedef _Float16 half2v __attribute__((ext_vector_type(2)));
    half2v v[N / 2];
    __device__ __forceinline__ void set(int j, _Float16 x) { v[j >> 1][j & 1] = x; }
    __device__ __forceinline__ float operator[](int j) const { return static_cast<float>(v[j >> 1][j & 1]); }
};


// DS: the channels of a row (D is the number this call handles, channels
// coff .. coff + D - 1).  With DS > D the channels are taken in npass calls
// (pass = 0, 1, ..); s_acc ([3][64] floats) carries the scalar gate's per-row
// channel sums and the prologue's row dots from one call to the next, and the
// prologue's earlier passes leave dq_hat, dk_hat in their workspace partial
// slots for the last pass to finish.
template <int D, int GATE, bool IN_F32, bool OUT_F32, bool PRO, bool KEEP, int DS = D, int ROUTE = 0>
__device__ __forceinline__ void grad_gate_body(int64_t T, int H, int64_t NC, const void* __restrict__ q_,
                                               const void* __restrict__ k_, const float* __restrict__ alpha,
                                               void* __restrict__ dq_, void* __restrict__ dk_,
                                               float* __restrict__ dalpha, ChunkWs ws, int pro, ChunkRange cr,
                                               char* smem, const GradPartials<D, IN_F32>& pk,
                                               const float* s_gam, float (&s_tot)[4][D], int coff = 0,
                                               int npass = 1, int pass = 0, float* s_acc = nullptr,
                                               int ahead = 0) {
    static_assert(DS == D || !KEEP, "channel passes keep the partials in the workspace");
    using L = GGateLayout<D, IN_F32>;
    using OpT = typename L::OpT;
    using InT = typename InType<IN_F32>::T;
    using OutT = typename InType<OUT_F32>::T;
    constexpr int NT = L::NT, NW = L::NW, LDC = L::LDC, RPP = 16;

    __shared__ float s_gs[CHUNK];
    __shared__ float s_red[NW];
    __shared__ float s_row[CHUNK];
    __shared__ float s_nrm[NW * 2 * RPP];  // prologue: row-dot partials
    __shared__ float s_rq[PRO ? CHUNK : 1], s_rk[PRO ? CHUNK : 1];  // prologue: reciprocal row norms

    OpT* dAs = reinterpret_cast<OpT*>(smem + L::DA);
    OpT* dPs = reinterpret_cast<OpT*>(smem + L::DP);
    OpT* dAT = reinterpret_cast<OpT*>(smem + L::DAT);
    OpT* dPT = reinterpret_cast<OpT*>(smem + L::DPT);
    OpT* QqT = reinterpret_cast<OpT*>(smem + L::QQT);
    OpT* KqT = reinterpret_cast<OpT*>(smem + L::KQT);
    OpT* KhT = reinterpret_cast<OpT*>(smem + L::KHT);
    float* SAf = reinterpret_cast<float*>(smem + L::SA);
    float* SBf = reinterpret_cast<float*>(smem + L::SB);
    float* SCf = reinterpret_cast<float*>(smem + L::SC);

    int64_t bh, c;
    range_block(cr, bh, c);
    const int64_t ch = bh * NC + c;
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh % H);
    const int64_t t0 = c * CHUNK;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int cc = tid % D, part = tid / D, r0 = part * RPP;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t tokstride = static_cast<int64_t>(H) * DS;
    const int64_t base = ((b * T + t0) * H + h) * DS + coff;
    const int64_t nvalid64 = T - t0;
    const int nvalid = nvalid64 < CHUNK ? static_cast<int>(nvalid64) : CHUNK;
    const InT* q = reinterpret_cast<const InT*>(q_);
    const InT* k = reinterpret_cast<const InT*>(k_);
    const OpT* gA = KEEP ? nullptr : static_cast<const OpT*>(ws.gA) + ch * CHUNK * CHUNK;
    const OpT* gP = KEEP ? nullptr : static_cast<const OpT*>(ws.gP) + ch * CHUNK * CHUNK;

    // ---------------- phase 0: G, block references, row operands, dA/dP ----------------
    // Every load of the phase is issued before any value is used, the token
    // values first (the scalar-gate scan needs only them).  Rows past the end
    // read the last row and are masked after the empty asm statement below: a
    // masking select on a loaded value may otherwise turn into a branch around
    // the load, which then waits for every load issued before it.
    const bool tok_ok = tid < nvalid;
    float at0 = 1.f, rq0 = 0.f, rk0 = 0.f;
    if (tid < CHUNK) {
        const int64_t tok = (b * T + t0 + (tok_ok ? tid : nvalid - 1)) * H + h;
        if constexpr (GATE == GATE_SCALAR) at0 = alpha[tok];
        if constexpr (PRO) {
            rq0 = ws.rq[tok];
            rk0 = ws.rk[tok];
        }
    }
    float G[RPP], kk[RPP], qq[RPP], al[RPP];
#pragma unroll
    for (int j = 0; j < RPP; ++j) {
        const int r = r0 + j;
        const int64_t e = base + (r < nvalid ? r : nvalid - 1) * tokstride + cc;
        kk[j] = to_f32(k[e]);
        qq[j] = to_f32(q[e]);
        if constexpr (GATE == GATE_CHANNEL) al[j] = alpha[e];
        else al[j] = 1.f;
    }
    // L2 prefetch for the workgroup `ahead` places later in the launch (on the
    // same XCD, as ahead is a multiple of 8): one dword per 128-byte line of
    // its first operands, k, alpha and N, issued after this stage's own loads.
    // The values are folded into tx, which is kept alive to the end, so the
    // loads are issued here and waited for only there.
    uint32_t tx = 0;
    if constexpr (!IN_F32 && DS == D) {
        const int64_t tb = static_cast<int64_t>(blockIdx.x) + ahead;
        if (ahead > 0 && tb < static_cast<int64_t>(gridDim.x)) {
            const uint32_t n = static_cast<uint32_t>(cr.n);
            const int64_t bh_t = tb / n, c_t = cr.lo + tb % n;
            const int64_t t0_t = c_t * CHUNK;
            const int64_t nv64 = T - t0_t;
            const int nv_t = nv64 < CHUNK ? static_cast<int>(nv64) : CHUNK;
            const int64_t base_t = (((bh_t / H) * T + t0_t) * H + bh_t % H) * D;
            const char* nw = reinterpret_cast<const char*>(ws.Nw) + (bh_t * NC + c_t) * CHUNK * CHUNK * 4;
            // lines: k rows (D/64 each), alpha rows (D/32 each; channel gate), N (128)
            constexpr int KL = D / 64, AL = GATE == GATE_CHANNEL ? D / 32 : 0, NL = CHUNK * (KL + AL) + 128;
#pragma unroll
            for (int l0 = 0; l0 < NL; l0 += NT) {
                const int line = l0 + tid;
                if (NL % NT == 0 || line < NL) {
                    const char* addr;
                    if (line < CHUNK * KL) {
                        const int r = line / KL < nv_t ? line / KL : nv_t - 1;
                        addr = reinterpret_cast<const char*>(k + base_t + r * tokstride) + (line % KL) * 128;
                    } else if (line < CHUNK * (KL + AL)) {
                        const int la = line - CHUNK * KL, r = la / AL < nv_t ? la / AL : nv_t - 1;
                        addr = reinterpret_cast<const char*>(alpha + base_t + r * tokstride) + (la % AL) * 128;
                    } else {
                        addr = nw + (line - CHUNK * (KL + AL)) * 128;
                    }
                    tx ^= *reinterpret_cast<const uint32_t*>(addr);
                }
            }
        }
    }
    asm volatile("" ::: "memory");
    if constexpr (GATE == GATE_SCALAR) {
        if (tid < CHUNK) {
            float g = tok_ok ? (PRO ? log2_alpha_logit(at0, pro) : log2_fast(at0)) : 0.f;
            s_row[tid] = tok_ok ? at0 : 1.f;
            s_gs[tid] = chunk_prefix_sum(g);
        }
    }
#pragma unroll
    for (int j = 0; j < RPP; ++j) {
        const bool ok = r0 + j < nvalid;
        kk[j] = ok ? kk[j] : 0.f;
        qq[j] = ok ? qq[j] : 0.f;
        if constexpr (GATE == GATE_CHANNEL) {
            // prologue: al stays the logit (the final dalpha needs it)
            al[j] = ok ? al[j] : 1.f;
            G[j] = ok ? (PRO ? log2_alpha_logit(al[j], pro) : log2_fast(al[j])) : 0.f;
        } else {
            G[j] = 0.f;
        }
    }
    if constexpr (PRO) {
        if (tid < CHUNK) {
            s_rq[tid] = rq0;
            s_rk[tid] = rk0;
        }
    }
    if constexpr (GATE == GATE_CHANNEL) {
#pragma unroll
        for (int j = 1; j < RPP; ++j) G[j] += G[j - 1];
        s_tot[part][cc] = G[RPP - 1];
    }
    // dA, dP (operand precision) into LDS, both orientations; Kh^T starts at
    // zero.  On chip: from this thread's accumulator-layout values (four rows of
    // a column), else from the workspace in 16-byte pieces of one row.
    if constexpr (KEEP) {
        using P = GradPartials<D, IN_F32>;
        const int itp = wid & 3;
#pragma unroll
        for (int k2 = 0; k2 < P::NPW; ++k2) {
            const int r = 16 * ((wid >> 2) + k2 * P::NHALF) + 4 * g4, i = 16 * itp + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) dAs[(r + e) * LDC + i] = pk.a[k2][e];
            *reinterpret_cast<typename P::V4*>(dAT + i * LDC + r) = pk.a[k2];
        }
#pragma unroll
        for (int t = 0; t < P::NTL; ++t) {
            const int tile = wid + t * NW, r = 16 * (tile / 4) + 4 * g4, i = 16 * (tile % 4) + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) dPs[(r + e) * LDC + i] = pk.p[t][e];
            *reinterpret_cast<typename P::V4*>(dPT + i * LDC + r) = pk.p[t];
        }
    } else {
        constexpr int EPV = 16 / static_cast<int>(sizeof(OpT));  // elements per piece
        constexpr int NV = CHUNK * CHUNK / EPV / NT;              // pieces per thread
        static_assert(CHUNK * CHUNK % (EPV * NT) == 0 && CHUNK % EPV == 0, "dA/dP pieces");
        uint4v ra[NV], rp[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            ra[v] = *reinterpret_cast<const uint4v*>(gA + (v * NT + tid) * EPV);
            rp[v] = *reinterpret_cast<const uint4v*>(gP + (v * NT + tid) * EPV);
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int e0 = (v * NT + tid) * EPV, r = e0 / CHUNK, i0 = e0 % CHUNK;
            *reinterpret_cast<uint4v*>(dAs + r * LDC + i0) = ra[v];
            *reinterpret_cast<uint4v*>(dPs + r * LDC + i0) = rp[v];
            const OpT* a = reinterpret_cast<const OpT*>(&ra[v]);
            const OpT* p = reinterpret_cast<const OpT*>(&rp[v]);
#pragma unroll
            for (int u = 0; u < EPV; ++u) {
                dAT[(i0 + u) * LDC + r] = a[u];
                dPT[(i0 + u) * LDC + r] = p[u];
            }
        }
    }
    {
        constexpr int NZ = D * LDC * static_cast<int>(sizeof(OpT)) / 16;
        static_assert(D * LDC * sizeof(OpT) % 16 == 0, "Kh^T in 16-byte pieces");
        uint4v* kz = reinterpret_cast<uint4v*>(KhT);
        const uint4v z = {0u, 0u, 0u, 0u};
        for (int e = tid; e < NZ; e += NT) kz[e] = z;
    }
    __syncthreads();
    if constexpr (PRO) {
        // prologue: q and k divided by their row norms
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            qq[j] *= fabsf(s_rq[r0 + j]);
            kk[j] *= fabsf(s_rk[r0 + j]);
        }
    }

    float carry = 0.f, glast = 0.f;
    if constexpr (GATE == GATE_CHANNEL) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const float t = s_tot[p][cc];
            carry += (p < part) ? t : 0.f;
            glast += t;
        }
#pragma unroll
        for (int j = 0; j < RPP; ++j) G[j] += carry;
    } else if constexpr (GATE == GATE_SCALAR) {
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            G[j] = s_gs[r0 + j];
            al[j] = s_row[r0 + j];
        }
        carry = part ? s_gs[r0 - 1] : 0.f;
        glast = s_gs[CHUNK - 1];
    }
    // exact-path flags: decay range of each diagonal block, max over channels
    int flags = 0;
    if constexpr (GATE != GATE_NONE) {
        float rho = carry - G[RPP - 1];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) rho = fmaxf(rho, __shfl_xor(rho, off));
        if (lane == 0) s_red[wid] = rho;  // each wave holds one block
    }
    __syncthreads();
    s_tot[part][cc] = G[RPP - 1];  // G at the last row of block `part` (0 without a gate)
    if constexpr (GATE != GATE_NONE) {
        constexpr int WPB = D / WAVE;
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            float rho = s_red[R * WPB];
#pragma unroll
            for (int w = 1; w < WPB; ++w) rho = fmaxf(rho, s_red[R * WPB + w]);
            if (!(rho <= L::RHO_MAX)) flags |= 1 << R;
        }
    }
    {
        // row operands Qq, Kq (reference = G before this thread's block), transposed
        float fq[RPP], kq_[RPP];
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            const float f = exp2_fast(G[j] - carry);
            fq[j] = qq[j] * f;
            kq_[j] = kk[j] * f;
        }
        store_run<OpT, RPP>(QqT + cc * LDC + r0, fq);
        store_run<OpT, RPP>(KqT + cc * LDC + r0, kq_);
    }
    // flagged diagonal blocks are excluded from the matrix-core products: their
    // Kh rows are zero in the row-side products (below), and their transposed
    // dA and dP blocks are zeroed for the column side; dA and dP themselves
    // keep the values the exact path reads
    if (flags) {
        for (int e = tid; e < 4 * 256; e += NT) {
            const int R = e / 256;
            if (!((flags >> R) & 1)) continue;
            const int r = 16 * R + (e % 256) / 16, i = 16 * R + e % 16;
            const OpT z = from_f32<OpT>(0.f);
            dAT[i * LDC + r] = z;
            dPT[i * LDC + r] = z;
        }
    }
    __syncthreads();

    // ---------------- phases R = 0..3 ----------------
    float Aq[RPP], Prow[RPP], Ccol[RPP];
#pragma unroll
    for (int j = 0; j < RPP; ++j) {
        Aq[j] = 0.f;
        Prow[j] = 0.f;
        Ccol[j] = 0.f;
    }
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        const float ref = R ? s_tot[R - 1][cc] : 0.f;
        if (part <= R) {
            float kh[RPP];
            const bool zero = (part == R) && ((flags >> R) & 1);
#pragma unroll
            for (int j = 0; j < RPP; ++j) kh[j] = zero ? 0.f : kk[j] * exp2_fast(ref - G[j]);
            store_run<OpT, RPP>(KhT + cc * LDC + r0, kh);
        }
        __syncthreads();
        // (a) dA_R Kh, (b) dP_R Kh: 16 x D each, k over 16(R+1) columns
        // (c) [dA_R^T | dP_R^T] [Qq_R ; Kq_R]: 16(R+1) x D, one 32-wide k step
        // Wave w takes column tile w of all of them (D / 16 tiles, one per wave):
        // a fixed set of products, so every read is issued before the first one
        // is used.
        static_assert(D / 16 == NW, "one column tile per wave");
        {
            const int ct = wid;
            const int nkq = (16 * (R + 1) + 31) / 32;  // a constant once the R loop is unrolled
            float4v acc[2];
#pragma unroll
            for (int isP = 0; isP < 2; ++isP) {
                const OpT* arow = (isP ? dPs : dAs) + (16 * R + l16) * LDC + 8 * g4;
                const OpT* brow = KhT + (16 * ct + l16) * LDC + 8 * g4;
                acc[isP] = zero4();
#pragma unroll
                for (int kq = 0; kq < 2; ++kq) {
                    if (kq < nkq) {
                        Frag<OpT> fa, fb;
                        fa.load(arow + 32 * kq);
                        fb.load(brow + 32 * kq);
                        mma(fa, fb, acc[isP]);
                    }
                }
            }
            float4v accc[4];
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                if (it > R) continue;
                Frag<OpT> fa, fb;
                // k < 16: dA^T and Qq; k >= 16: dP^T and Kq (lane groups 0,1 vs 2,3)
                const int i = 16 * it + l16, kr = 16 * R + 8 * (g4 & 1);
                fa.load((g4 < 2 ? dAT : dPT) + i * LDC + kr);
                fb.load((g4 < 2 ? QqT : KqT) + (16 * ct + l16) * LDC + kr);
                accc[it] = zero4();
                mma(fa, fb, accc[it]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                SAf[(4 * g4 + e) * D + 16 * ct + l16] = acc[0][e];
                SBf[(4 * g4 + e) * D + 16 * ct + l16] = acc[1][e];
            }
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                if (it > R) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) SCf[(16 * it + 4 * g4 + e) * D + 16 * ct + l16] = accc[it][e];
            }
        }
        __syncthreads();
        if (part == R) {
#pragma unroll
            for (int j = 0; j < RPP; ++j) {
                Aq[j] += SAf[j * D + cc];
                Prow[j] += SBf[j * D + cc];
            }
        }
        // column side, scaled by Fh = 2^(ref(R) - G) (a flagged diagonal block
        // contributes nothing here; its exact terms are added below)
        if (part < R || (part == R && !((flags >> R) & 1))) {
#pragma unroll
            for (int j = 0; j < RPP; ++j) Ccol[j] += SCf[(r0 + j) * D + cc] * exp2_fast(ref - G[j]);
        }
        __syncthreads();
    }
    // row-side factor Fq = 2^(G - ref(own block))
#pragma unroll
    for (int j = 0; j < RPP; ++j) {
        const float f = exp2_fast(G[j] - carry);
        Aq[j] *= f;
        Prow[j] *= f;
    }
    // exact diagonal blocks (fp32, pair factors 2^(G_r - G_i) <= 1)
    if ((flags >> part) & 1) {
        const OpT* sAr = dAs + r0 * LDC + r0;
        const OpT* sPr = dPs + r0 * LDC + r0;
#pragma unroll
        for (int jr = 0; jr < RPP; ++jr) {
#pragma unroll
            for (int ji = 0; ji <= jr; ++ji) {
                const float E = exp2_fast(G[jr] - G[ji]);
                const float da = to_f32(sAr[jr * LDC + ji]), dp = (ji < jr) ? to_f32(sPr[jr * LDC + ji]) : 0.f;
                Aq[jr] += da * kk[ji] * E;
                Prow[jr] += dp * kk[ji] * E;
                Ccol[ji] += (da * qq[jr] + dp * kk[jr]) * E;
            }
        }
    }

    // ---------------- combine ----------------
    float dG[RPP];
    float lastsum = 0.f;  // sum_r k_r . dKb_r . 2^(G_last - G_r): goes to the last row
    {
        OutT* dq = reinterpret_cast<OutT*>(dq_);
        OutT* dk = reinterpret_cast<OutT*>(dk_);
        // every partial is loaded before the first store (the stores could
        // alias them as far as the compiler knows); fp16 partials two rows to a
        // register, which keeps this phase within the register file
        PairRows<OpT, RPP> pq, pkt, pkb;
        using P = GradPartials<D, IN_F32>;
        if constexpr (KEEP && P::QREG) {
            // on chip: this thread's accumulator-layout values into the exchange,
            // then its 16 rows of column cc out of it, in 16-byte pieces
            using V4 = typename P::V4;
            constexpr int EPC = L::EPC, NPC = L::NPC;
            OpT* X = reinterpret_cast<OpT*>(smem + L::XR);  // [3][D][64]: dQt, dKt, dKb
            __syncthreads();  // the R loop's reads of SA..SC and the exact path's of dA, dP are done
            {
                const int col = 16 * wid + l16;
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int o = xoff<EPC, NPC>(col, 16 * r4 + 4 * g4);
                    *reinterpret_cast<V4*>(X + o) = pk.q[r4];
                    *reinterpret_cast<V4*>(X + 2 * CHUNK * D + o) = pk.kb[r4];
                }
                const int rt = wid & 3, half = wid >> 2;
#pragma unroll
                for (int ii = 0; ii < P::NIT; ++ii) {
                    const int c2 = 16 * (half + P::NHALF * ii) + l16;
                    *reinterpret_cast<V4*>(X + CHUNK * D + xoff<EPC, NPC>(c2, 16 * rt + 4 * g4)) = pk.kt[ii];
                }
            }
            __syncthreads();
            static_assert(RPP % EPC == 0, "whole pieces per thread");
#pragma unroll
            for (int pc = 0; pc < RPP / EPC; ++pc) {
                const int o = xoff<EPC, NPC>(cc, r0 + pc * EPC);
                const uint4v vq = *reinterpret_cast<const uint4v*>(X + o);
                const uint4v vt = *reinterpret_cast<const uint4v*>(X + CHUNK * D + o);
                const uint4v vb = *reinterpret_cast<const uint4v*>(X + 2 * CHUNK * D + o);
                const OpT* eq = reinterpret_cast<const OpT*>(&vq);
                const OpT* et = reinterpret_cast<const OpT*>(&vt);
                const OpT* eb = reinterpret_cast<const OpT*>(&vb);
#pragma unroll
                for (int u = 0; u < EPC; ++u) {
                    pq.set(pc * EPC + u, eq[u]);
                    pkt.set(pc * EPC + u, et[u]);
                    pkb.set(pc * EPC + u, eb[u]);
                }
            }
            if constexpr (PRO) __syncthreads();  // the prologue's dq_hat / dk_hat below overlap the exchange
        } else {
            const OpT* gQt = static_cast<const OpT*>(ws.gQt) + ch * CHUNK * DS + coff;
            const OpT* gKb = static_cast<const OpT*>(ws.gKb) + ch * CHUNK * DS + coff;
#pragma unroll
            for (int j = 0; j < RPP; ++j) {
                pq.set(j, gQt[(r0 + j) * DS + cc]);
                pkb.set(j, gKb[(r0 + j) * DS + cc]);
            }
            if constexpr (KEEP && P::TLDS) {
                // dKt from LDS past this stage's buffers (written in the first stage)
                const OpT* X = reinterpret_cast<const OpT*>(smem + L::BYTES);
#pragma unroll
                for (int pc = 0; pc < RPP / L::EPC; ++pc) {
                    const uint4v vt = *reinterpret_cast<const uint4v*>(X + xoff<L::EPC, L::NPC>(cc, r0 + pc * L::EPC));
                    const OpT* et = reinterpret_cast<const OpT*>(&vt);
#pragma unroll
                    for (int u = 0; u < L::EPC; ++u) pkt.set(pc * L::EPC + u, et[u]);
                }
            } else {
                const OpT* gKt = static_cast<const OpT*>(ws.gKt) + ch * CHUNK * DS + coff;
#pragma unroll
                for (int j = 0; j < RPP; ++j) pkt.set(j, gKt[(r0 + j) * DS + cc]);
            }
        }
        if constexpr (!PRO) {
#pragma unroll
            for (int j = 0; j < RPP; ++j) {
                const int r = r0 + j;
                const float E = exp2_fast(G[j]), Eb = exp2_fast(glast - G[j]);
                const float gq = pq[j] * E, gkt = pkt[j] * E, gkb = pkb[j] * Eb;
                const float dqv = gq + Aq[j];
                const float dkv = gkt + gkb + Prow[j] + Ccol[j];
                dG[j] = qq[j] * dqv + kk[j] * (gkt - gkb + Prow[j] - Ccol[j]);
                lastsum += kk[j] * gkb;
                if (r < nvalid) {
                    dq[base + r * tokstride + cc] = from_f32<OutT>(dqv);
                    dk[base + r * tokstride + cc] = from_f32<OutT>(dkv);
                }
            }
        } else {
            // prologue: back through x / |x|: (dx_hat - x_hat (x_hat . dx_hat)) / |x|
            // (only dx_hat / eps where the norm was clamped).  dq_hat and dk_hat
            // wait in LDS (the product buffers are free now) while the row dots
            // are summed, which keeps them out of the register file.
            float* sQ = SCf;                                     // [64][D] fp32
            float* sK = reinterpret_cast<float*>(smem + L::DA);  // [64][D] fp32 over dA .. dP^T
            static_assert(CHUNK * D * 4 <= L::QQT - L::DA, "dk_hat must fit over dA .. dP^T");
            float dot[2 * RPP];
#pragma unroll
            for (int j = 0; j < RPP; ++j) {
                const float E = exp2_fast(G[j]), Eb = exp2_fast(glast - G[j]);
                const float gq = pq[j] * E, gkt = pkt[j] * E, gkb = pkb[j] * Eb;
                const float dqv = gq + Aq[j];
                const float dkv = gkt + gkb + Prow[j] + Ccol[j];
                dG[j] = qq[j] * dqv + kk[j] * (gkt - gkb + Prow[j] - Ccol[j]);
                lastsum += kk[j] * gkb;
                sQ[(r0 + j) * D + cc] = dqv;
                sK[(r0 + j) * D + cc] = dkv;
                dot[j] = qq[j] * dqv;
                dot[RPP + j] = kk[j] * dkv;
            }
            part_row_sums32<D>(dot, s_nrm);
            if (npass > 1) {
                // channel passes: a row's dots run over every pass (the earlier
                // passes' sums first)
                float* pdot = s_acc + CHUNK;  // [2][64]
                if (pass > 0) {
#pragma unroll
                    for (int j = 0; j < RPP; ++j) {
                        dot[j] = pdot[r0 + j] + dot[j];
                        dot[RPP + j] = pdot[CHUNK + r0 + j] + dot[RPP + j];
                    }
                }
                __syncthreads();
                if (cc == 0) {
#pragma unroll
                    for (int j = 0; j < RPP; ++j) {
                        pdot[r0 + j] = dot[j];
                        pdot[CHUNK + r0 + j] = dot[RPP + j];
                    }
                }
                if (pass + 1 < npass) {
                    // dq_hat, dk_hat wait in this pass's dQt, dKb slots (read above)
                    OpT* hq = static_cast<OpT*>(ws.gQt) + ch * CHUNK * DS + coff;
                    OpT* hk = static_cast<OpT*>(ws.gKb) + ch * CHUNK * DS + coff;
#pragma unroll
                    for (int j = 0; j < RPP; ++j) {
                        hq[(r0 + j) * DS + cc] = from_f32<OpT>(sQ[(r0 + j) * D + cc]);
                        hk[(r0 + j) * DS + cc] = from_f32<OpT>(sK[(r0 + j) * D + cc]);
                    }
                }
            }
            if (npass == 1 || pass + 1 == npass) {
#pragma unroll
                for (int j = 0; j < RPP; ++j) {
                    const int r = r0 + j;
                    if (r >= nvalid) continue;
                    const float rq = s_rq[r], rk = s_rk[r];
                    const float dqv = sQ[r * D + cc], dkv = sK[r * D + cc];
                    const float gq = (rq > 0.f) ? (dqv - qq[j] * dot[j]) * rq : -dqv * rq;
                    const float gk = (rk > 0.f) ? (dkv - kk[j] * dot[RPP + j]) * rk : -dkv * rk;
                    dq[base + r * tokstride + cc] = from_f32<OutT>(gq);
                    dk[base + r * tokstride + cc] = from_f32<OutT>(gk);
                }
            }
            if (npass > 1 && pass + 1 == npass) {
                // the earlier passes' channels, from their waiting dq_hat, dk_hat and
                // their q and k rows normalised again
#pragma unroll 1
                for (int pp = 0; pp + 1 < npass; ++pp) {
                    const int64_t bp = base - coff + D * pp;
                    const OpT* hq = static_cast<const OpT*>(ws.gQt) + ch * CHUNK * DS + D * pp;
                    const OpT* hk = static_cast<const OpT*>(ws.gKb) + ch * CHUNK * DS + D * pp;
#pragma unroll 2
                    for (int j = 0; j < RPP; ++j) {
                        const int r = r0 + j;
                        if (r >= nvalid) continue;
                        const float rq = s_rq[r], rk = s_rk[r];
                        const float qh = to_f32(q[bp + r * tokstride + cc]) * fabsf(rq);
                        const float kh = to_f32(k[bp + r * tokstride + cc]) * fabsf(rk);
                        const float dqv = to_f32(hq[r * DS + cc]), dkv = to_f32(hk[r * DS + cc]);
                        const float gq = (rq > 0.f) ? (dqv - qh * dot[j]) * rq : -dqv * rq;
                        const float gk = (rk > 0.f) ? (dkv - kh * dot[RPP + j]) * rk : -dkv * rk;
                        dq[bp + r * tokstride + cc] = from_f32<OutT>(gq);
                        dk[bp + r * tokstride + cc] = from_f32<OutT>(gk);
                    }
                }
            }
        }
    }
    if constexpr (GATE != GATE_NONE) {
        // gradient w.r.t. G (natural-log units) -> reverse cumsum over the chunk -> dalpha
        // part sums of dG and of the last-row term, for the carries between parts
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < RPP; ++j) psum += dG[j];
        __syncthreads();
        s_tot[part][cc] = psum;
        __syncthreads();
        float later = 0.f;  // sum of dG over rows after this thread's block
#pragma unroll
        for (int p = 0; p < 4; ++p) later += (p > part) ? s_tot[p][cc] : 0.f;
        __syncthreads();
        s_tot[part][cc] = lastsum;
        __syncthreads();
        float ltot = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p) ltot += s_tot[p][cc];
        // the last row (and so every row, through the reverse cumsum) also gets
        // d/dG_last of Kb's 2^G_last and of gamma: sum_r k.dKb.2^(Gl-G) + gamma.dgamma
        const float gl_term = ltot + exp2_fast(glast) * (KEEP ? s_gam[cc] : ws.gGam[ch * DS + coff + cc]);
        float run = later + gl_term;
        float dg[RPP];
#pragma unroll
        for (int j = RPP - 1; j >= 0; --j) {
            run += dG[j];
            dg[j] = run;
        }
        if constexpr (GATE == GATE_CHANNEL) {
#pragma unroll
            for (int j = 0; j < RPP; ++j) {
                const int r = r0 + j;
                if (r < nvalid)
                    dalpha[base + r * tokstride + cc] = PRO ? dlogit_from_dlog(dg[j], al[j], pro) : dg[j] / al[j];
            }
        } else {
            // scalar gate: sum over channels, in a fixed order: each wave sums
            // its 64 channels of a row, then the D / 64 wave sums of the row
            // are added in channel order (s_tot is free again after ltot)
            float* s_wsum = &s_tot[0][0];  // [D / 64][CHUNK]
            static_assert((D / 64) * CHUNK <= 4 * D, "wave sums fit s_tot");
            __syncthreads();
#pragma unroll
            for (int j = 0; j < RPP; ++j) {
                float x = dg[j];
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
                if (lane == 0) s_wsum[(cc >> 6) * CHUNK + r0 + j] = x;
            }
            __syncthreads();
            if (tid < CHUNK) {
                float srow = s_wsum[tid];
#pragma unroll
                for (int w = 1; w < D / 64; ++w) srow += s_wsum[w * CHUNK + tid];
                if (npass > 1) {  // channel passes: the earlier passes' sum first
                    if (pass > 0) srow = s_acc[tid] + srow;
                    if (pass + 1 < npass) s_acc[tid] = srow;
                }
                if (pass + 1 == npass && tid < nvalid) {
                    float a1 = alpha[(b * T + t0 + tid) * H + h];
                    dalpha[(b * T + t0 + tid) * H + h] = PRO ? dlogit_from_dlog(srow, a1, pro) : srow / a1;
                }
            }
        }
    }
    asm volatile("" ::"v"(tx));  // the prefetch loads end here at the latest
}

// The error route's terms between the stages when the first stage's partials
// stay on chip (d = 128, fp16 operands): dKt -= dE S^T on its LDS copy past the
// second stage's buffers, dP -= strict_tril(dE U^T) on the dP tiles this wave
// holds in pk, each rounded to operand precision exactly as the workspace
// route's read-modify-writes round them; dE and the scale gradient's partial
// row as in cler_post_body.
template <int D, bool IN_F32>
__device__ __forceinline__ void cler_post_onchip(int64_t T, int H, int64_t NC, const ChunkWs& ws,
                                                 const float* __restrict__ beta, const float* __restrict__ lam,
                                                 const void* __restrict__ dh_, float* __restrict__ partial,
                                                 ChunkRange cr, char* smem, GradPartials<D, IN_F32>& pk) {
    using P = GradPartials<D, IN_F32>;
    using GL = GGateLayout<D, IN_F32>;
    using Lc = ClerLayout<D, IN_F32>;
    using OpT = typename Lc::OpT;
    using V4 = typename P::V4;
    constexpr int NT = 4 * D, NW = NT / 64, KQ = D / 32, LDE = Lc::LDE;
    static_assert(P::TLDS && !IN_F32, "dKt on chip in LDS");
    static_assert(D / 16 == NW, "one state-row tile of dKt per wave");
    static_assert(Lc::POST_BYTES <= GL::BYTES, "dE below the dKt copy");
    const OpT* sE = reinterpret_cast<const OpT*>(smem);
    OpT* X = reinterpret_cast<OpT*>(smem + GL::BYTES);  // dKt, the second stage's exchange layout

    int64_t bh, c;
    range_block(cr, bh, c);
    const int64_t ch = bh * NC + c;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const OpT* U = reinterpret_cast<const OpT*>(ws.Usave) + ch * CHUNK * D;
    const OpT* Ss = reinterpret_cast<const OpT*>(ws.Ssnap) + ch * D * D;
    const int dt = wid;
    Frag<OpT> fs[KQ];
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) fs[kq].load(Ss + ((dt * KQ + kq) * 64 + lane) * 8);

    cler_build_dE<D, IN_F32, NT>(T, H, NC, ws, beta, lam, dh_, partial, cr, smem);

    // dKt -= dE S^T: state-row tile dt = wid, four position tiles
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
        for (int rt = 0; rt < 4; ++rt) {
            V4* piece = reinterpret_cast<V4*>(X + xoff<GL::EPC, GL::NPC>(16 * dt + l16, 16 * rt + 4 * g4));
            V4 v = *piece;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = from_f32<OpT>(to_f32(v[e]) - acc[rt][e]);
            *piece = v;
        }
    }
    // dP -= strict_tril(dE U^T) on this wave's tiles wid + NW t of pk.p
#pragma unroll
    for (int t = 0; t < P::NTL; ++t) {
        const int tile = wid + NW * t, at = tile / 4, xt = tile % 4;
        if (xt <= at) {
            float4v acc = zero4();
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq) {
                Frag<OpT> fe, fu;
                fe.load(sE + (16 * at + l16) * LDE + 32 * kq + 8 * g4);
                fu.load(U + ((xt * KQ + kq) * 64 + lane) * 8);
                mma(fe, fu, acc);
            }
            const int x = 16 * xt + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int a = 16 * at + 4 * g4 + e;
                if (x < a) pk.p[t][e] = from_f32<OpT>(to_f32(pk.p[t][e]) - acc[e]);
            }
        }
    }
}

// Both gradient stages for one chunk in one workgroup: the partials grad_lin
// writes are read back by the same workgroup, from the L2, after a barrier that
// makes them visible; the LDS buffer is shared.  With the error-routing
// epilogue (CLER) the write errors' own terms (cler_post_body, which edits the
// dKt and dP partials and writes the chunk's scale-gradient partial row) run
// between the two, behind barriers of their own.
template <int D, int GATE, bool IN_F32, bool OUT_F32, bool PRO, bool CLER>
__global__ __launch_bounds__(4 * D) void grads_kernel(int64_t T, int H, int64_t NC, float scale,
                                                      const void* __restrict__ q_, const void* __restrict__ k_,
                                                      const void* __restrict__ v_, const float* __restrict__ beta,
                                                      const float* __restrict__ alpha, const void* __restrict__ dO_,
                                                      const void* __restrict__ dh_, const float* __restrict__ lam,
                                                      void* __restrict__ dq_, void* __restrict__ dk_,
                                                      void* __restrict__ dv_, float* __restrict__ dbeta,
                                                      float* __restrict__ dalpha, ChunkWs ws, int pro,
                                                      ChunkRange cr, float* __restrict__ partial, int ahead) {
    constexpr int LB = GLinLayout<D, IN_F32>::BYTES, GB = GGateLayout<D, IN_F32>::BYTES;
    static_assert(!CLER || ClerLayout<D, IN_F32>::POST_BYTES <= (LB > GB ? LB : GB), "LDS of the CLER terms");
    // The partials stay on chip on the value route, and on the error route at
    // d = 128 with fp16 operands, whose terms then edit them there; otherwise
    // the error route's terms edit them in the workspace between the stages.
    constexpr bool KEEP = !CLER || (GradPartials<D, IN_F32>::TLDS && !IN_F32);
    // d = 128: dKt waits past the second stage's buffers
    constexpr int GBX = GB + ((KEEP && GradPartials<D, IN_F32>::TLDS) ? CHUNK * D * (IN_F32 ? 4 : 2) : 0);
    __shared__ __attribute__((aligned(16))) char smem[LB > GBX ? LB : GBX];
    __shared__ float s_gam[KEEP ? D : 1];
    __shared__ float s_tot[4][D];  // per-part column sums, used by both stages in turn
    GradPartials<D, IN_F32> pk;
    grad_lin_body<D, GATE, IN_F32, OUT_F32, PRO, KEEP, false, CLER>(T, H, NC, scale, k_, v_, beta, alpha, dO_, dh_,
                                                                     lam, dv_, dbeta, ws, pro, cr, smem, pk, s_gam,
                                                                     s_tot);
    __syncthreads();
    if constexpr (CLER) {
        if constexpr (KEEP) cler_post_onchip<D, IN_F32>(T, H, NC, ws, beta, lam, dh_, partial, cr, smem, pk);
        else cler_post_body<D, IN_F32, 4 * D>(T, H, NC, ws, beta, lam, dh_, partial, cr, smem);
        __syncthreads();
    }
    grad_gate_body<D, GATE, IN_F32, OUT_F32, PRO, KEEP, D, CLER>(T, H, NC, q_, k_, alpha, dq_, dk_, dalpha, ws, pro,
                                                                  cr, smem, pk, s_gam, s_tot, 0, 1, 0, nullptr, ahead);
}

// fp32 operands at d = 128, where one workgroup's LDS cannot hold either stage:
// the stages as two kernels with every partial in the workspace.  The first
// reads its row operands from global memory; the second takes the channels in
// two passes of 64 (its block products are independent per channel).
template <int GATE, bool OUT_F32, bool CLER, bool PRO>
__global__ __launch_bounds__(512) void grad_lin_split_kernel(int64_t T, int H, int64_t NC, float scale,
                                                             const void* __restrict__ k_, const void* __restrict__ v_,
                                                             const float* __restrict__ beta,
                                                             const float* __restrict__ alpha,
                                                             const void* __restrict__ dO_, const void* __restrict__ dh_,
                                                             const float* __restrict__ lam, void* __restrict__ dv_,
                                                             float* __restrict__ dbeta, ChunkWs ws, int pro,
                                                             ChunkRange cr, float* __restrict__ partial) {
    constexpr int LB = GLinLayout<128, true, true>::BYTES;
    static_assert(!CLER || ClerLayout<128, true>::POST_BYTES <= LB, "LDS of the CLER terms");
    __shared__ __attribute__((aligned(16))) char smem[LB];
    __shared__ float s_tot[4][128];
    GradPartials<128, true> pk;
    grad_lin_body<128, GATE, true, OUT_F32, PRO, false, true>(T, H, NC, scale, k_, v_, beta, alpha, dO_, dh_, lam,
                                                              dv_, dbeta, ws, pro, cr, smem, pk, nullptr, s_tot);
    if constexpr (CLER) {
        __syncthreads();
        cler_post_body<128, true, 512>(T, H, NC, ws, beta, lam, dh_, partial, cr, smem);
    }
}

template <int GATE, bool OUT_F32, bool PRO>
__global__ __launch_bounds__(256) void grad_gate_split_kernel(int64_t T, int H, int64_t NC, const void* __restrict__ q_,
                                                              const void* __restrict__ k_,
                                                              const float* __restrict__ alpha, void* __restrict__ dq_,
                                                              void* __restrict__ dk_, float* __restrict__ dalpha,
                                                              ChunkWs ws, int pro, ChunkRange cr) {
    __shared__ __attribute__((aligned(16))) char smem[GGateLayout<64, true>::BYTES];
    __shared__ float s_tot[4][64];
    __shared__ float s_acc[3 * CHUNK];
    GradPartials<64, true> pk;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        if (pass) __syncthreads();
        grad_gate_body<64, GATE, true, OUT_F32, PRO, false, 128>(T, H, NC, q_, k_, alpha, dq_, dk_, dalpha, ws, pro,
                                                                 cr, smem, pk, nullptr, s_tot, 64 * pass, 2, pass,
                                                                 s_acc);
    }
}

template <int GATE, bool OUT_F32>
static hipError_t launch_grads_split(int64_t B, int64_t T, int H, int64_t NC, float scale, const void* q,
                                     const void* k, const void* v, const float* beta, const float* alpha,
                                     const void* dO, const void* dh, const float* lam, void* dq, void* dk, void* dv,
                                     float* dbeta, float* dalpha, const ChunkWs& ws, int pro, ChunkRange cr,
                                     bool cler, float* partial, int, hipStream_t stream) {
    const int64_t nblk = B * H * cr.n;
    if (nblk == 0) return hipSuccess;
#define GDR_LIN_SPLIT(C, P)                                                                                      \
    hipLaunchKernelGGL((grad_lin_split_kernel<GATE, OUT_F32, C, P>), dim3((unsigned)nblk), dim3(512), 0, stream, T, \
                       H, NC, scale, k, v, beta, alpha, dO, dh, lam, dv, dbeta, ws, pro, cr, partial)
    if (cler) {
        if (pro) GDR_LIN_SPLIT(true, true);
        else GDR_LIN_SPLIT(true, false);
    } else {
        if (pro) GDR_LIN_SPLIT(false, true);
        else GDR_LIN_SPLIT(false, false);
    }
#undef GDR_LIN_SPLIT
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (pro)
        hipLaunchKernelGGL((grad_gate_split_kernel<GATE, OUT_F32, true>), dim3((unsigned)nblk), dim3(256), 0, stream, T,
                           H, NC, q, k, alpha, dq, dk, dalpha, ws, pro, cr);
    else
        hipLaunchKernelGGL((grad_gate_split_kernel<GATE, OUT_F32, false>), dim3((unsigned)nblk), dim3(256), 0, stream,
                           T, H, NC, q, k, alpha, dq, dk, dalpha, ws, pro, cr);
    return hipGetLastError();
}

template <int D, int GATE, bool IN_F32, bool OUT_F32>
static hipError_t launch_grads_t(int64_t B, int64_t T, int H, int64_t NC, float scale, const void* q,
                                 const void* k, const void* v, const float* beta, const float* alpha,
                                 const void* dO, const void* dh, const float* lam, void* dq, void* dk, void* dv,
                                 float* dbeta, float* dalpha, const ChunkWs& ws, int pro, ChunkRange cr,
                                 bool cler, float* partial, int ahead, hipStream_t stream) {
    const int64_t nblk = B * H * cr.n;
    if (nblk == 0) return hipSuccess;
#define GDR_GRADS(P, C)                                                                                              \
    hipLaunchKernelGGL((grads_kernel<D, GATE, IN_F32, OUT_F32, P, C>), dim3((unsigned)nblk), dim3(4 * D), 0, stream, \
                       T, H, NC, scale, q, k, v, beta, alpha, dO, dh, lam, dq, dk, dv, dbeta, dalpha, ws, pro, cr,    \
                       partial, ahead)
    if (cler) {
        if (pro) GDR_GRADS(true, true);
        else GDR_GRADS(false, true);
    } else {
        if (pro) GDR_GRADS(true, false);
        else GDR_GRADS(false, false);
    }
#undef GDR_GRADS
    return hipGetLastError();
}

template <int D, int GATE>
static hipError_t launch_grads_g(bool in_f32, bool out_f32, int64_t B, int64_t T, int H, int64_t NC, float scale,
                                 const void* q, const void* k, const void* v, const float* beta,
                                 const float* alpha, const void* dO, const void* dh, const float* lam, void* dq,
                                 void* dk, void* dv, float* dbeta, float* dalpha, const ChunkWs& ws, int pro,
                                 ChunkRange cr, bool cler, float* partial, int ahead, hipStream_t stream) {
#define GDR_GR_ARGS B, T, H, NC, scale, q, k, v, beta, alpha, dO, dh, lam, dq, dk, dv, dbeta, dalpha, ws, pro, cr, \
                    cler, partial, ahead, stream
    if (in_f32) {
        if constexpr (D == 64) {
            if (out_f32) return launch_grads_t<D, GATE, true, true>(GDR_GR_ARGS);
            return launch_grads_t<D, GATE, true, false>(GDR_GR_ARGS);
        }
        if constexpr (D == 128) {
            if (out_f32) return launch_grads_split<GATE, true>(GDR_GR_ARGS);
            return launch_grads_split<GATE, false>(GDR_GR_ARGS);
        }
    }
    if (out_f32) return launch_grads_t<D, GATE, false, true>(GDR_GR_ARGS);
    return launch_grads_t<D, GATE, false, false>(GDR_GR_ARGS);
#undef GDR_GR_ARGS
}

hipError_t launch_grads(int D, int gate, bool in_f32, bool out_f32, int64_t B, int64_t T, int H, int64_t NC,
                        float scale, const void* q, const void* k, const void* v, const float* beta,
                        const float* alpha, const void* dO, const void* dh, const float* lam, void* dq, void* dk,
                        void* dv, float* dbeta, float* dalpha, const ChunkWs& ws, int pro, ChunkRange cr,
                        bool cler, float* partial, int ahead, hipStream_t stream) {
#define GDR_GR_ARGS in_f32, out_f32, B, T, H, NC, scale, q, k, v, beta, alpha, dO, dh, lam, dq, dk, dv, dbeta, \
                    dalpha, ws, pro, cr, cler, partial, ahead, stream
    if (D == 64) {
        if (gate == GATE_NONE) return launch_grads_g<64, GATE_NONE>(GDR_GR_ARGS);
        if (gate == GATE_SCALAR) return launch_grads_g<64, GATE_SCALAR>(GDR_GR_ARGS);
        return launch_grads_g<64, GATE_CHANNEL>(GDR_GR_ARGS);
    }
    if (gate == GATE_NONE) return launch_grads_g<128, GATE_NONE>(GDR_GR_ARGS);
    if (gate == GATE_SCALAR) return launch_grads_g<128, GATE_SCALAR>(GDR_GR_ARGS);
    return launch_grads_g<128, GATE_CHANNEL>(GDR_GR_ARGS);
#undef GDR_GR_ARGS
}

// ---------------------------------------------------------------------------
// CLVR: dlam[c] = sum over tokens of dh[., c] * v[., c]  (c = h*dv + j).
// Pass 1: nseg token segments, one partial per (segment, channel).
// Pass 2: sum the partials of each channel in a fixed order (deterministic).
// ---------------------------------------------------------------------------
// CLVR scale gradient, dlam[c] = sum over (b, t) of dh[b,t,c] * v[b,t,c], in two
// deterministic passes.  Pass 1: segment y of the token range, thread x owns
// VEC consecutive columns (one 16-byte load per row of each operand).
template <bool IN_F32>
__global__ __launch_bounds__(256) void clvr_dlam_partial(int64_t BT, int HD, int64_t nseg, const void* __restrict__ dh_,
                                                         const void* __restrict__ v_, float* __restrict__ partial) {
    using InT = typename InType<IN_F32>::T;
    constexpr int VEC = 16 / sizeof(InT);
    const InT* dh = reinterpret_cast<const InT*>(dh_);
    const InT* v = reinterpret_cast<const InT*>(v_);
    const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * VEC;
    const int64_t seg = blockIdx.y;
    if (c0 >= HD) return;
    const int64_t per = (BT + nseg - 1) / nseg;
    const int64_t t0 = seg * per, t1 = t0 + per < BT ? t0 + per : BT;
    float s[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) s[e] = 0.f;
    // rows in groups of RB: every load of a group is issued before the first
    // product (rows past the end re-read the last row and are masked after),
    // and the products are added in row order
    constexpr int RB = 8;
#pragma unroll 1
    for (int64_t t = t0; t < t1; t += RB) {
        float4v rd[RB], rv[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t tr = t + r < t1 ? t + r : t1 - 1;
            rd[r] = *reinterpret_cast<const float4v*>(dh + tr * HD + c0);
            rv[r] = *reinterpret_cast<const float4v*>(v + tr * HD + c0);
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const InT* pd = reinterpret_cast<const InT*>(&rd[r]);
            const InT* pv = reinterpret_cast<const InT*>(&rv[r]);
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                s[e] = t + r < t1 ? __builtin_fmaf(to_f32(pd[e]), to_f32(pv[e]), s[e]) : s[e];
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) partial[seg * HD + c0 + e] = s[e];
}

// Pass 2: 64 columns per workgroup; thread (column c, group g) sums segments
// g, g + 4, ...; the four group sums are added in a fixed order.
__global__ __launch_bounds__(256) void clvr_dlam_final(int HD, int64_t nseg, const float* __restrict__ partial,
                                                       float* __restrict__ dlam) {
    __shared__ float red[4][64];
    const int cl = threadIdx.x & 63, g = threadIdx.x >> 6;
    const int64_t c = static_cast<int64_t>(blockIdx.x) * 64 + cl;
    float s = 0.f;
    if (c < HD) {
        // segments g, g + 4, ... added in that order, eight loads in flight at a
        // time (indices past the end re-read the last segment and are masked)
        constexpr int SB = 8;
#pragma unroll 1
        for (int64_t seg = g; seg < nseg; seg += 4 * SB) {
            float x[SB];
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                const int64_t sg = seg + 4 * u < nseg ? seg + 4 * u : nseg - 1;
                x[u] = partial[sg * HD + c];
            }
            asm volatile("" ::: "memory");
#pragma unroll
            for (int u = 0; u < SB; ++u) s = seg + 4 * u < nseg ? s + x[u] : s;
        }
    }
    red[g][cl] = s;
    __syncthreads();
    if (g == 0 && c < HD) dlam[c] = ((red[0][cl] + red[1][cl]) + red[2][cl]) + red[3][cl];
}

hipError_t launch_clvr_dlam(bool in_f32, int64_t BT, int H, int D, const void* dh, const void* v,
                            float* dlam, float* partial, int64_t nseg, hipStream_t stream) {
    const int HD = H * D;
    const int vec = in_f32 ? 4 : 8;
    const dim3 g1((HD / vec + 255) / 256, (unsigned)nseg);
    if (in_f32)
        hipLaunchKernelGGL((clvr_dlam_partial<true>), g1, dim3(256), 0, stream, BT, HD, nseg, dh, v, partial);
    else
        hipLaunchKernelGGL((clvr_dlam_partial<false>), g1, dim3(256), 0, stream, BT, HD, nseg, dh, v, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_dlam_final(HD, nseg, partial, dlam, stream);
}

hipError_t launch_dlam_final(int HD, int64_t nseg, const float* partial, float* dlam, hipStream_t stream) {
    hipLaunchKernelGGL(clvr_dlam_final, dim3((HD + 63) / 64), dim3(256), 0, stream, HD, nseg, partial, dlam);
    return hipGetLastError();
}

}  // namespace gdr
