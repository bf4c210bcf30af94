// gdr_gdn2.hip -- Gated DeltaNet-2: separate erase and write gates.
//
// The popular article on the study (its Gated DeltaNet-2 paragraph) describes
// this member in words only: erasing old content and writing new content are
// decoupled and steered by two gates computed independently from the token, an
// erase gate choosing the regions of the memory to clear and a write gate the
// regions to write; equal gates fall back to Kimi Delta Attention.  The regions
// are read as key channels (rows of S), the gates as dk-vectors e_t, w_t:
//     S_t = (I - (e_t*k_t) k_t^T) Diag(alpha_t) S_{t-1} + (w_t*k_t) v_t^T
//     o_t = scale * S_t^T q_t
// With e = w = beta 1 this is the KDA step.
//
// Chunked form (chunk start state S, G_r the in-chunk cumulative log2 decay,
// Kt = K*2^G, Qt = Q*2^G, Eh = (e*K)*2^-G, Wh = (w*K)*2^-G, Eb = (e*K)*2^(G_last-G),
// Wb = (w*K)*2^(G_last-G), all row-wise; P the rows of the predictions S'^T k):
//     M_e = strict_tril(Kt Eh^T)   M_w = strict_tril(Kt Wh^T)
//     A_e = tril(Qt Eh^T)          A_w = tril(Qt Wh^T)
//     P   = N (Kt S + M_w V),      N = (I + M_e)^-1
//     O   = Qt S + A_w V - A_e P
//     S'  = Diag(2^G_last) S + Wb^T V - Eb^T P
// Only P depends on S, through W = N Kt.  The intra-chunk kernel writes the
// operands of the fp32 state pass, with U = -P = Ut - W S:
//     W = N Kt, Ut = -N M_w V, Qt, KbT = Eb^T, A = A_e, gam, X = Wb^T V, Y = A_w V
// and the pass runs U = Ut - W S, O = scale (Qt S + A U + Y),
// S <- Diag(gam) S + KbT U + X.
//
// Two intra-chunk kernels compute these operands.  For bf16 inputs
// (gdn2_intra_h_kernel) every product takes fp16 operands with fp32
// accumulation, the operands are staged once in LDS, and the stored W, Ut, Qt,
// KbT, A are fp16 (the operand precision of the KDA path); X and Y stay fp32.
// For fp32 inputs (gdn2_intra_kernel) everything is fp32 and the block pairs
// are formed pair by pair from the inputs: its LDS budget has no room for fp32
// staging.  In both, a diagonal block whose decay range exceeds what the
// operands carry (2^8 for fp16, 2^60 for fp32) is computed without the split
// into row and column factors.
#include <type_traits>

#include "gdr_common.hpp"
#include "gdr_launch.hpp"

namespace gdr {

namespace {

constexpr int NT2 = 512;  // threads of the intra-chunk kernel

// wave-wide maximum
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

// Eight consecutive input elements held as loaded (bf16: four registers), so
// that many loads can be in flight at once; converted at use.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
    uint4 r;
    __device__ __forceinline__ void load(const bf16_t* p) { r = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ float at(int i) const {
        const uint32_t word = (i >> 1) == 0 ? r.x : (i >> 1) == 1 ? r.y : (i >> 1) == 2 ? r.z : r.w;
        return __uint_as_float((i & 1) ? (word & 0xffff0000u) : (word << 16));
    }
};
template <> struct Raw8<float> {
    float4v a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = reinterpret_cast<const float4v*>(p)[0];
        b = reinterpret_cast<const float4v*>(p)[1];
    }
    __device__ __forceinline__ float at(int i) const { return i < 4 ? a[i] : b[i - 4]; }
};

template <typename OpT>
__device__ __forceinline__ void set_frag(Frag<OpT>& f, const float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = from_f32<OpT>(x[i]);
}

// fp32 inputs.  Range of the decay factors: every product of a row factor
// 2^(G_r - ref) and a column factor 2^(ref - G_j) uses a reference between the
// two (the end of the column block for blocks below the diagonal, so both
// factors are at most 1; the start of the block on the diagonal, where the
// column factor is at most 2^rho for the block's decay range rho).  A diagonal
// block whose range exceeds 60 (in log2) is computed pair by pair with
// 2^(G_r - G_j) formed directly.
template <int D, int GATE, bool IN_F32>
__global__ __launch_bounds__(NT2) void gdn2_intra_kernel(int64_t T, int H, int64_t NC, const void* __restrict__ q_,
                                                         const void* __restrict__ k_, const void* __restrict__ v_,
                                                         const float* __restrict__ erase,
                                                         const float* __restrict__ write,
                                                         const float* __restrict__ alpha, ChunkWs ws,
                                                         ChunkRange cr) {
    using InT = typename InType<IN_F32>::T;
    // operand precision (as in the KDA path): fp16 for bf16 inputs, fp32 for
    // fp32 inputs -- of the C x C blocks (a diagonal block whose decay range is
    // too wide for fp16 is computed pair by pair), the products with V, and the
    // operands the state pass reads (W, Ut, Qt, KbT, A); the solve's block
    // updates take fp32 operands
    using OpT = typename std::conditional<IN_F32, float, _Float16>::type;
    constexpr int NW = NT2 / WAVE;   // waves
    constexpr int P = NT2 / D;       // row parts of the channel-per-thread layout
    constexpr int RPP = CHUNK / P;   // rows per part
    constexpr int NCT = D / 16;      // 16-column tiles of a [..][D] matrix
    constexpr int LT = CHUNK + 4;    // row stride of the transposed [D][64] arrays (conflict-free columns)
    constexpr int BUF = CHUNK * D > D * LT ? CHUNK * D : D * LT;

    // sM: M_e, M_w, A_e, A_w [64][64]; sA: G [64][D], then Eb^T and V^T [D][64],
    // then M_w V and Vt [64][D]; sB: Wb^T [D][64], then Kt and W [64][D]
    __shared__ __attribute__((aligned(16))) float sM[4][CHUNK * CHUNK];
    __shared__ __attribute__((aligned(16))) float sA[BUF];
    __shared__ __attribute__((aligned(16))) float sB[BUF];
    __shared__ float s_tot[P][D];

    int64_t bh, c;  // the chunks of the range cr of every (batch, head)
    range_block(cr, bh, c);
    const int64_t ch = bh * NC + c;
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh % H);
    const int64_t t0 = c * CHUNK;
    const int nvalid = static_cast<int>(T - t0 < CHUNK ? T - t0 : CHUNK);
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int l16 = lane & 15, kg = 8 * (lane >> 4);
    const InT* q = reinterpret_cast<const InT*>(q_);
    const InT* k = reinterpret_cast<const InT*>(k_);
    const InT* v = reinterpret_cast<const InT*>(v_);
    // element offset of row r (rows past the sequence read the first row; their
    // values are zeroed by a factor, so loads need no branch)
    auto rowoff = [&](int r) -> int64_t { return ((b * T + t0 + (r < nvalid ? r : 0)) * H + h) * D; };

    // ---- phase 1: G, the in-chunk inclusive cumulative log2 decay, per channel
    {
        float4v* z4 = reinterpret_cast<float4v*>(&sM[0][0]);
        for (int i = tid; i < 4 * CHUNK * CHUNK / 4; i += NT2) z4[i] = zero4();
    }
    const int cc = tid % D, part = tid / D;
    {
        float av[RPP];
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            const int64_t e = rowoff(part * RPP + j) + cc;
            if constexpr (GATE == GATE_CHANNEL) av[j] = alpha[e];
            else if constexpr (GATE == GATE_SCALAR) av[j] = alpha[e / D];
            else av[j] = 1.f;
        }
        float g = 0.f, G[RPP];
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            const bool ok = part * RPP + j < nvalid;  // rows past the sequence decay by nothing
            g += (GATE != GATE_NONE && ok) ? log2_fast(av[j]) : 0.f;
            G[j] = g;
        }
        s_tot[part][cc] = g;
        __syncthreads();
        float carry = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) carry += (p < part) ? s_tot[p][cc] : 0.f;
#pragma unroll
        for (int j = 0; j < RPP; ++j) sA[(part * RPP + j) * D + cc] = G[j] + carry;
    }
    __syncthreads();
    const float* sG = sA;

    // ---- phase 2: the four C x C matrices, 16 x 16 block pairs (R, J), J <= R:
    // the diagonal blocks first (waves 0-3), the six below the diagonal after
    {
        const int pairR[10] = {0, 1, 2, 3, 1, 2, 3, 2, 3, 3};
        const int pairJ[10] = {0, 1, 2, 3, 0, 1, 2, 0, 1, 0};
        for (int pi = wid; pi < 10; pi += NW) {
            const int R = pairR[pi], J = pairJ[pi];
            bool exact = false;
            if (R == J) {
                float rho = 0.f;
                for (int c2 = lane; c2 < D; c2 += WAVE)
                    rho = fmaxf(rho, sG[(16 * R) * D + c2] - sG[(16 * R + 15) * D + c2]);
                // fp16 operands carry a column factor up to 2^8 (as in the KDA
                // kernel), fp32 ones up to 2^60
                exact = wave_max(rho) > (sizeof(OpT) == 2 ? 8.f : 60.f);
            }
            const int refrow = R == J ? 16 * R : 16 * J + 15;
            const int rr = 16 * R + l16, jj = 16 * J + l16;
            if (!exact) {
                float4v aMe = zero4(), aMw = zero4(), aAe = zero4(), aAw = zero4();
                const float mr = rr < nvalid ? 1.f : 0.f, mj = jj < nvalid ? 1.f : 0.f;
                const int64_t tr = rowoff(rr), tj = rowoff(jj);
                constexpr int NKQ = D / 32;
                Raw8<InT> rk[NKQ], rq[NKQ], rkj[NKQ];
                Raw8<float> re[NKQ], rw[NKQ];
#pragma unroll
                for (int kq = 0; kq < NKQ; ++kq) {
                    const int c0 = 32 * kq + kg;
                    rk[kq].load(k + tr + c0);
                    rq[kq].load(q + tr + c0);
                    rkj[kq].load(k + tj + c0);
                    re[kq].load(erase + tj + c0);
                    rw[kq].load(write + tj + c0);
                }
#pragma unroll
                for (int kq = 0; kq < NKQ; ++kq) {
                    const int c0 = 32 * kq + kg;
                    float xk[8], xq[8], ye[8], yw[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float ref = sG[refrow * D + c0 + i];
                        const float fr = mr * exp2_fast(sG[rr * D + c0 + i] - ref);
                        const float fc = mj * exp2_fast(ref - sG[jj * D + c0 + i]) * rkj[kq].at(i);
                        xk[i] = rk[kq].at(i) * fr;
                        xq[i] = rq[kq].at(i) * fr;
                        ye[i] = re[kq].at(i) * fc;
                        yw[i] = rw[kq].at(i) * fc;
                    }
                    Frag<OpT> Ak, Aq, Be, Bw;
                    set_frag(Ak, xk);
                    set_frag(Aq, xq);
                    set_frag(Be, ye);
                    set_frag(Bw, yw);
                    mma(Ak, Be, aMe);
                    mma(Ak, Bw, aMw);
                    mma(Aq, Be, aAe);
                    mma(Aq, Bw, aAw);
                }
                // lane: column jj, rows 16R + 4(lane / 16) + e
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * R + 4 * (lane >> 4) + e;
                    const bool keepM = J < R || jj < r, keepA = J < R || jj <= r;
                    sM[0][r * CHUNK + jj] = keepM ? aMe[e] : 0.f;
                    sM[1][r * CHUNK + jj] = keepM ? aMw[e] : 0.f;
                    sM[2][r * CHUNK + jj] = keepA ? aAe[e] : 0.f;
                    sM[3][r * CHUNK + jj] = keepA ? aAw[e] : 0.f;
                }
            } else {
                // diagonal block with a large decay range: 2^(G_r - G_j) per pair.
                // lane: row rr, columns 16R + 4(lane / 16) + i, i < 4
                const int jb = 16 * R + 4 * (lane >> 4);
                float me[4] = {0.f, 0.f, 0.f, 0.f}, mw[4] = {0.f, 0.f, 0.f, 0.f};
                float ae[4] = {0.f, 0.f, 0.f, 0.f}, aw[4] = {0.f, 0.f, 0.f, 0.f};
                if (rr < nvalid) {
                    const int64_t tr = rowoff(rr);
                    for (int c2 = 0; c2 < D; ++c2) {
                        const float gr = sG[rr * D + c2];
                        const float kr = to_f32(k[tr + c2]), qr = to_f32(q[tr + c2]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int j = jb + i;
                            if (j <= rr) {
                                const int64_t tj = rowoff(j) + c2;
                                const float f = exp2_fast(gr - sG[j * D + c2]);
                                const float kj = to_f32(k[tj]);
                                const float ej = erase[tj] * kj * f;
                                const float wj = write[tj] * kj * f;
                                me[i] += kr * ej;
                                mw[i] += kr * wj;
                                ae[i] += qr * ej;
                                aw[i] += qr * wj;
                            }
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = jb + i;
                    sM[0][rr * CHUNK + j] = j < rr ? me[i] : 0.f;
                    sM[1][rr * CHUNK + j] = j < rr ? mw[i] : 0.f;
                    sM[2][rr * CHUNK + j] = j <= rr ? ae[i] : 0.f;
                    sM[3][rr * CHUNK + j] = j <= rr ? aw[i] : 0.f;
                }
            }
        }
    }
    __syncthreads();

    // ---- phase 3: row-wise operands.  Wb into sB; Kt and Eb in registers
    OpT* Qt = static_cast<OpT*>(ws.Qt) + ch * CHUNK * D;
    OpT* KbT = static_cast<OpT*>(ws.KbT) + ch * D * CHUNK;
    float kt[RPP], eb[RPP];
    {
        float kv[RPP], ev[RPP], wv[RPP];
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            const int64_t e = rowoff(part * RPP + j) + cc;
            kv[j] = to_f32(k[e]);
            ev[j] = erase[e];
            wv[j] = write[e];
        }
        const float gl = sG[(CHUNK - 1) * D + cc];  // rows past the sequence carry the last decay
        if (part == 0) ws.gam[ch * D + cc] = exp2_fast(gl);
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            const int r = part * RPP + j;
            const float m = r < nvalid ? 1.f : 0.f;
            kv[j] *= m;
            const float gr = sG[r * D + cc];
            const float fl = exp2_fast(gl - gr);
            kt[j] = kv[j] * exp2_fast(gr);
            eb[j] = ev[j] * kv[j] * fl;
            sB[cc * LT + r] = wv[j] * kv[j] * fl;  // Wb^T [D][64], row stride LT
        }
        // Qt in fragment order: runs of eight channels of one row
        constexpr int NQ = CHUNK * D / 8 / NT2;
        float xq[NQ][8];
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int task = tid + i * NT2, r = task / (D / 8), c0 = 8 * (task % (D / 8));
            load8f(q + rowoff(r) + c0, xq[i]);
        }
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int task = tid + i * NT2, r = task / (D / 8), c0 = 8 * (task % (D / 8));
            const float m = r < nvalid ? 1.f : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) xq[i][e] *= m * exp2_fast(sG[r * D + c0 + e]);
            store_run<OpT, 8>(Qt + frag_off<D>(r, c0), xq[i]);
        }
        // A = A_e in fragment order
        OpT* A = static_cast<OpT*>(ws.A) + ch * CHUNK * CHUNK;
        for (int run = tid; run < CHUNK * CHUNK / 8; run += NT2) {
            const int r = run / (CHUNK / 8), j0 = 8 * (run % (CHUNK / 8));
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = sM[2][r * CHUNK + j0 + e];
            store_run<OpT, 8>(A + frag_off<CHUNK>(r, j0), x);
        }
    }
    __syncthreads();  // G is read for the last time
    // KbT = Eb^T in fragment order: Eb staged transposed over G, runs of eight tokens
#pragma unroll
    for (int j = 0; j < RPP; ++j) sA[cc * LT + part * RPP + j] = eb[j];
    __syncthreads();
    for (int task = tid; task < D * CHUNK / 8; task += NT2) {
        const int c2 = task / (CHUNK / 8), r0 = 8 * (task % (CHUNK / 8));
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = sA[c2 * LT + r0 + e];
        store_run<OpT, 8>(KbT + frag_off<CHUNK>(c2, r0), x);
    }
    __syncthreads();
    // V (fp32) over Eb^T
    {
        constexpr int NV = CHUNK * D / 8 / NT2;
        float x[NV][8];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int p = tid + i * NT2, r = p / (D / 8), c0 = 8 * (p % (D / 8));
            load8f(v + rowoff(r) + c0, x[i]);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int p = tid + i * NT2, r = p / (D / 8), c0 = 8 * (p % (D / 8));
            const float m = r < nvalid ? 1.f : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) sA[(c0 + e) * LT + r] = m * x[i][e];  // V^T [D][64], row stride LT
        }
    }
    __syncthreads();

    // ---- X = Wb^T V [D][D] (contraction over the 64 rows), accumulator order
    {
        float* X = ws.X + ch * D * D;
        for (int tile = wid; tile < NCT * NCT; tile += NW) {
            const int mt = tile / NCT, nt = tile % NCT;
            float4v acc = zero4();
#pragma unroll
            for (int kq = 0; kq < CHUNK / 32; ++kq) {
                float xa[8], xb[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 32 * kq + kg + i;
                    xa[i] = sB[(16 * mt + l16) * LT + r];
                    xb[i] = sA[(16 * nt + l16) * LT + r];
                }
                Frag<OpT> fa, fb;
                set_frag(fa, xa);
                set_frag(fb, xb);
                mma(fa, fb, acc);
            }
            *reinterpret_cast<float4v*>(X + ((mt * NCT + nt) * WAVE + lane) * 4) = acc;
        }
    }

    // ---- Y = A_w V and M_w V [64][D] (contraction over the 64 columns)
    constexpr int MT = CHUNK / 16 * NCT;  // 16 x 16 tiles of a [64][D] result
    constexpr int MPW = MT / NW;          // per wave
    static_assert(MT % NW == 0, "tiles per wave");
    float4v mwv[MPW];
    {
        float* Y = ws.Y + ch * CHUNK * D;
#pragma unroll
        for (int i = 0; i < MPW; ++i) {
            const int tile = wid + NW * i;
            const int mt = tile / NCT, nt = tile % NCT;
            float4v ay = zero4(), am = zero4();
#pragma unroll
            for (int kq = 0; kq < CHUNK / 32; ++kq) {
                float xw[8], xm[8], xb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = 32 * kq + kg + e;
                    xw[e] = sM[3][(16 * mt + l16) * CHUNK + j];
                    xm[e] = sM[1][(16 * mt + l16) * CHUNK + j];
                    xb[e] = sA[(16 * nt + l16) * LT + j];
                }
                Frag<OpT> fw, fm, fb;
                set_frag(fw, xw);
                set_frag(fm, xm);
                set_frag(fb, xb);
                mma(fw, fb, ay);
                mma(fm, fb, am);
            }
            *reinterpret_cast<float4v*>(Y + ((mt * NCT + nt) * WAVE + lane) * 4) = ay;
            mwv[i] = am;
        }
    }
    __syncthreads();  // every read of Wb (sB) and V (sA) is done
    // right-hand sides of the solve: Kt into sB, M_w V into sA (row-major)
#pragma unroll
    for (int j = 0; j < RPP; ++j) sB[(part * RPP + j) * D + cc] = kt[j];
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
        const int tile = wid + NW * i;
        const int mt = tile / NCT, nt = tile % NCT;
#pragma unroll
        for (int e = 0; e < 4; ++e) sA[(16 * mt + 4 * (lane >> 4) + e) * D + 16 * nt + l16] = mwv[i][e];
    }
    __syncthreads();

    // ---- phase 5: (I + M_e) Z = [Kt | M_w V] for Z = [W | Vt], in place, by
    // 16-row blocks: block R first takes the products of the solved rows above
    // it, M_e[R, <16R] Z[<16R] (fp32 matrix cores, one 16-column tile per wave),
    // then is solved by forward substitution inside the block (one column per
    // thread).  Column t < D lives in sB, the others in sA.
    auto zat = [&](int r, int col) -> float& { return col < D ? sB[r * D + col] : sA[r * D + col - D]; };
#pragma unroll
    for (int R = 0; R < CHUNK / 16; ++R) {
        if (R > 0) {
            for (int ct = wid; ct < 2 * NCT; ct += NW) {
                float4v acc = zero4();
                const int col = 16 * ct + l16;
#pragma unroll
                for (int kq = 0; kq < (16 * R + 31) / 32; ++kq) {
                    float xa[8], xb[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int j = 32 * kq + kg + i;
                        xa[i] = j < 16 * R ? sM[0][(16 * R + l16) * CHUNK + j] : 0.f;
                        xb[i] = j < 16 * R ? zat(j, col) : 0.f;
                    }
                    Frag<float> fa, fb;
                    set_frag(fa, xa);
                    set_frag(fb, xb);
                    mma(fa, fb, acc);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) zat(16 * R + 4 * (lane >> 4) + e, col) -= acc[e];
            }
            __syncthreads();
        }
        if (tid < 2 * D) {
            float z[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) z[i] = zat(16 * R + i, tid);
#pragma unroll
            for (int i = 1; i < 16; ++i) {
                const int r = 16 * R + i;
                float m[16];
#pragma unroll
                for (int j4 = 0; j4 < (i + 3) / 4; ++j4) {
                    const float4v x = *reinterpret_cast<const float4v*>(&sM[0][r * CHUNK + 16 * R + 4 * j4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) m[4 * j4 + e] = x[e];
                }
                float acc = z[i];
#pragma unroll
                for (int j = 0; j < i; ++j) acc -= m[j] * z[j];
                z[i] = acc;
            }
#pragma unroll
            for (int i = 1; i < 16; ++i) zat(16 * R + i, tid) = z[i];
        }
        __syncthreads();
    }

    // ---- outputs: W (sB) in fragment order, Ut = -Vt (sA) in accumulator order
    OpT* W = static_cast<OpT*>(ws.W) + ch * CHUNK * D;
    for (int task = tid; task < CHUNK * D / 8; task += NT2) {
        const int r = task / (D / 8), c0 = 8 * (task % (D / 8));
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = sB[r * D + c0 + e];
        store_run<OpT, 8>(W + frag_off<D>(r, c0), x);
    }
    OpT* Ut = static_cast<OpT*>(ws.Ut) + ch * CHUNK * D;
    for (int task = tid; task < CHUNK / 4 * D; task += NT2) {
        const int r = 4 * (task / D), n = task % D;
        float4v u;
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = -sA[(r + e) * D + n];
        store4<OpT>(Ut + cfrag_off<D>(r, n), u);
    }
}

// The intra-chunk transform for fp16 operands (bf16 inputs), staged once in LDS.
//
// Decay factors.  With ref(R) = G at the last row before block R (0 for R = 0)
// and end(J) = G at the last row of block J, every pair factor 2^(G_r - G_j)
// (j <= r) splits into per-element factors of at most 1 and one per-channel
// scale per block pair:
//     2^(G_r - G_j) = a_r * c_RJ * b_j,   a_r = 2^(G_r - ref(R)),
//     b_j = 2^(end(J) - G_j),             c_RJ = 2^(ref(R) - end(J)).
// c_RJ = 1 for J = R - 1, <= 1 further below the diagonal, and on the diagonal
// it is 2^rho_R (rho_R the block's whole decay), the only factor above 1: a
// block with rho_R > 8 is computed exactly instead, from running products of
// alpha.  The row operands k a and q a are staged in fp32 and the column
// operands (e k) b and (w k) b in fp16, so each block pair only scales its row
// operands by c_RJ before the single rounding to fp16.  All exponents are <= 0
// apart from the diagonal scale, so no chunk is too wide for the fp32 range.
//
// Solve.  N_RR = (I + M_e[R,R])^-1 for the four diagonal blocks, one lane per
// column, then for each block row R (in order)
//     Z_R = N_RR (rhs_R - sum_{K<R} M_e[R,K] Z_K),  rhs = [Kt | M_w V],
// on fp32 matrix cores.  Each wave owns whole 16-column tiles of Z and keeps
// its Z_K in registers: the lane layout of the 16x16x4 fp32 product gives lane
// group g the reduction indices 4g .. 4g+3, the rows of the accumulator it
// holds, so Z_K feeds the next product directly and block rows need no barrier.
template <int D, int GATE>
struct Gdn2HLayout {
    static constexpr int P = NT2 / D;       // row parts (one channel per thread)
    static constexpr int RPP = CHUNK / P;   // rows per part: 8 or 16, inside one block
    static constexpr int NCT = D / 16;      // 16-column tiles of a [..][D] matrix
    static constexpr int LKR = D + 4;       // fp32 rows of the staged row operands
    static constexpr int LEH = D + 8;       // fp16 rows of the staged column operands
    static constexpr int LT32 = CHUNK + 4;  // fp32 rows of [D][64] Kt^T
    static constexpr int LT16 = CHUNK + 8;  // fp16 rows of [D][64] V^T and Wb^T
    static constexpr int LM32 = CHUNK + 4;  // fp32 rows of M_e
    static constexpr int LM16 = CHUNK + 8;  // fp16 rows of A_e, M_w, A_w
    static constexpr int LN = 20;           // fp32 rows of the diagonal inverses
    // region A, block pairs: k a and q a (fp32), (e k) b and (w k) b (fp16)
    static constexpr int KR = 0;
    static constexpr int QR = KR + CHUNK * LKR * 4;
    static constexpr int EH = QR + CHUNK * LKR * 4;
    static constexpr int WH = EH + CHUNK * LEH * 2;
    static constexpr int PAIRS_END = WH + CHUNK * LEH * 2;
    // region A, after the block pairs: Kt^T (fp32), V^T and Wb^T (fp16; Wb^T's
    // space then stages W in fragment order), Qt in fragment order
    static constexpr int KTT = 0;
    static constexpr int VT = KTT + D * LT32 * 4;
    static constexpr int WBT = VT + D * LT16 * 2;
    static constexpr int QTS = WBT + D * LT16 * 2;
    static constexpr int SOLVE_END = QTS + CHUNK * D * 2;
    static constexpr int AREG = PAIRS_END > SOLVE_END ? PAIRS_END : SOLVE_END;
    // the four C x C matrices and the diagonal inverses
    static constexpr int ME = AREG;
    static constexpr int AE = ME + CHUNK * LM32 * 4;
    static constexpr int MW = AE + CHUNK * LM16 * 2;
    static constexpr int AW = MW + CHUNK * LM16 * 2;
    static constexpr int NINV = AW + CHUNK * LM16 * 2;
    static constexpr int BYTES = NINV + 4 * 16 * LN * 4;
    static_assert(CHUNK * D * 2 <= D * LT16 * 2, "W staging fits in Wb^T's space");
    static_assert(RPP == 8 || RPP == 16, "a part lies inside one 16-row block");
};

template <int D, int GATE>
__global__ __launch_bounds__(NT2) void gdn2_intra_h_kernel(int64_t T, int H, int64_t NC, const void* __restrict__ q_,
                                                           const void* __restrict__ k_, const void* __restrict__ v_,
                                                           const float* __restrict__ erase,
                                                           const float* __restrict__ write,
                                                           const float* __restrict__ alpha, ChunkWs ws,
                                                           ChunkRange cr) {
    using L = Gdn2HLayout<D, GATE>;
    using OpT = _Float16;
    constexpr int NW = NT2 / WAVE, P = L::P, RPP = L::RPP, NCT = L::NCT;
    constexpr int LKR = L::LKR, LEH = L::LEH, LT32 = L::LT32, LT16 = L::LT16;
    constexpr int LM32 = L::LM32, LM16 = L::LM16, LN = L::LN;
    constexpr float RHO_MAX = 8.f;  // in-block decay (log2) that fp16 row operands carry

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    __shared__ float s_tot[P][D];
    __shared__ __attribute__((aligned(16))) float s_c[7][D];  // block-pair scales
    __shared__ float s_red[NW][4];

    float* sKR = reinterpret_cast<float*>(smem + L::KR);
    float* sQR = reinterpret_cast<float*>(smem + L::QR);
    OpT* sEH = reinterpret_cast<OpT*>(smem + L::EH);
    OpT* sWH = reinterpret_cast<OpT*>(smem + L::WH);
    float* sKTT = reinterpret_cast<float*>(smem + L::KTT);
    OpT* sVT = reinterpret_cast<OpT*>(smem + L::VT);
    OpT* sWBT = reinterpret_cast<OpT*>(smem + L::WBT);
    OpT* sWS = reinterpret_cast<OpT*>(smem + L::WBT);
    OpT* sQTS = reinterpret_cast<OpT*>(smem + L::QTS);
    float* sME = reinterpret_cast<float*>(smem + L::ME);
    OpT* sAE = reinterpret_cast<OpT*>(smem + L::AE);
    OpT* sMW = reinterpret_cast<OpT*>(smem + L::MW);
    OpT* sAW = reinterpret_cast<OpT*>(smem + L::AW);
    float* sN = reinterpret_cast<float*>(smem + L::NINV);

    int64_t bh, c;  // the chunks of the range cr of every (batch, head)
    range_block(cr, bh, c);
    const int64_t ch = bh * NC + c;
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh % H);
    const int64_t t0 = c * CHUNK;
    const int nvalid = static_cast<int>(T - t0 < CHUNK ? T - t0 : CHUNK);
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4, kg = 8 * g4;
    const int cc = tid % D, part = tid / D, r0 = part * RPP, R0 = r0 / 16;
    const bf16_t* q = reinterpret_cast<const bf16_t*>(q_);
    const bf16_t* k = reinterpret_cast<const bf16_t*>(k_);
    const bf16_t* v = reinterpret_cast<const bf16_t*>(v_);
    const int64_t tokstride = static_cast<int64_t>(H) * D;
    const int64_t base = ((b * T + t0) * H + h) * D;  // element (row 0, channel 0) of this chunk
    // rows past the sequence read the last valid row (in bounds) and are zeroed
    auto rowoff = [&](int r) -> int64_t { return base + (r < nvalid ? r : nvalid - 1) * tokstride; };

    // ---- loads: every input of this thread's rows, issued back to back
    float kk[RPP], qq[RPP], vv[RPP], ee[RPP], ww[RPP], G[RPP];
#pragma unroll
    for (int j = 0; j < RPP; ++j) {
        const int64_t e = rowoff(r0 + j) + cc;
        kk[j] = to_f32(k[e]);
        qq[j] = to_f32(q[e]);
        vv[j] = to_f32(v[e]);
        ee[j] = erase[e];
        ww[j] = write[e];
        if constexpr (GATE == GATE_CHANNEL) G[j] = alpha[e];
        else if constexpr (GATE == GATE_SCALAR) G[j] = alpha[e / D];
        else G[j] = 1.f;
    }
    // G: inclusive cumulative log2 decay inside the chunk; rows past the
    // sequence decay by nothing
#pragma unroll
    for (int j = 0; j < RPP; ++j) {
        const bool ok = r0 + j < nvalid;
        kk[j] = ok ? kk[j] : 0.f;
        qq[j] = ok ? qq[j] : 0.f;
        vv[j] = ok ? vv[j] : 0.f;
        ee[j] = ok ? ee[j] : 0.f;
        ww[j] = ok ? ww[j] : 0.f;
        G[j] = (GATE != GATE_NONE && ok) ? log2_fast(G[j]) : 0.f;
    }
#pragma unroll
    for (int j = 1; j < RPP; ++j) G[j] += G[j - 1];
    s_tot[part][cc] = G[RPP - 1];
    __syncthreads();
    // bend[R] = G at the last row of block R (this thread's channel)
    float carry = 0.f, bend[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const float t = s_tot[p][cc];
        carry += p < part ? t : 0.f;
#pragma unroll
        for (int R = 0; R < 4; ++R) bend[R] += (p * RPP < 16 * (R + 1)) ? t : 0.f;
    }
#pragma unroll
    for (int j = 0; j < RPP; ++j) G[j] += carry;
    const float refm = R0 > 0 ? bend[R0 - 1] : 0.f, refp = bend[R0], glast = bend[3];

    // ---- element-wise operands
    float kt[RPP], qt[RPP], wb[RPP];
    {
        const float eref = exp2_fast(refm), efl = exp2_fast(glast - refp);
        float eb[RPP];
#pragma unroll
        for (int j = 0; j < RPP; ++j) {
            const int r = r0 + j;
            const float a = exp2_fast(G[j] - refm), bj = exp2_fast(refp - G[j]);
            sKR[r * LKR + cc] = kk[j] * a;
            sQR[r * LKR + cc] = qq[j] * a;
            const float ek = ee[j] * kk[j], wk = ww[j] * kk[j];
            sEH[r * LEH + cc] = from_f32<OpT>(ek * bj);
            sWH[r * LEH + cc] = from_f32<OpT>(wk * bj);
            const float E = a * eref, fl = bj * efl;  // 2^G, 2^(G_last - G)
            kt[j] = kk[j] * E;
            qt[j] = qq[j] * E;
            eb[j] = ek * fl;
            wb[j] = wk * fl;
        }
        // Kb^T = Eb^T (A operand of Kb^T U: rows channel, k = position), runs of 8
        OpT* KbT = static_cast<OpT*>(ws.KbT) + ch * D * CHUNK;
#pragma unroll
        for (int j = 0; j < RPP; j += 8) store_run<OpT, 8>(KbT + frag_off<CHUNK>(cc, r0 + j), eb + j);
        if (part == 0) {
            ws.gam[ch * D + cc] = exp2_fast(glast);
            // block-pair scales: (2,0), (3,0), (3,1) below the diagonal, then the
            // four diagonal blocks
            s_c[0][cc] = exp2_fast(bend[1] - bend[0]);
            s_c[1][cc] = exp2_fast(bend[2] - bend[0]);
            s_c[2][cc] = exp2_fast(bend[2] - bend[1]);
            s_c[3][cc] = exp2_fast(-bend[0]);
            s_c[4][cc] = exp2_fast(bend[0] - bend[1]);
            s_c[5][cc] = exp2_fast(bend[1] - bend[2]);
            s_c[6][cc] = exp2_fast(bend[2] - bend[3]);
        }
        // widest in-block decay of the wave's channels, per block
        float rho[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) rho[R] = wave_max((R > 0 ? bend[R - 1] : 0.f) - bend[R]);
        if (lane == 0) {
#pragma unroll
            for (int R = 0; R < 4; ++R) s_red[wid][R] = rho[R];
        }
    }
    __syncthreads();
    int flags = 0;  // bit R: diagonal block R is computed exactly
    if constexpr (GATE != GATE_NONE) {
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            float rho = s_red[0][R];
#pragma unroll
            for (int w = 1; w < NW; ++w) rho = fmaxf(rho, s_red[w][R]);
            if (!(rho <= RHO_MAX)) flags |= 1 << R;  // NaN-safe
        }
    }

    // ---- the four C x C matrices by 16 x 16 block pairs (R, J), J <= R.
    // Pairs 0-3 are the diagonal, 4-6 need a scale below the diagonal, 7-9 not.
    {
#pragma unroll 1
        for (int pi = wid; pi < 10; pi += NW) {
            // (R, J, scale row): 0-3 (p, p, 3 + p); 4-6 (2, 0, 0), (3, 0, 1),
            // (3, 1, 2); 7-9 (p - 6, p - 7, none)
            const int R = pi < 4 ? pi : pi < 7 ? (pi == 4 ? 2 : 3) : pi - 6;
            const int J = pi < 4 ? pi : pi < 7 ? (pi == 6 ? 1 : 0) : pi - 7;
            const int si = pi < 4 ? 3 + pi : pi < 7 ? pi - 4 : -1;
            if (R == J && ((flags >> R) & 1)) continue;  // exact path below
            float4v aMe = zero4(), aMw = zero4(), aAe = zero4(), aAw = zero4();
            const int rr = 16 * R + l16, jj = 16 * J + l16;
#pragma unroll
            for (int kq = 0; kq < D / 32; ++kq) {
                const int c0 = 32 * kq + kg;
                const float4v k0 = *reinterpret_cast<const float4v*>(sKR + rr * LKR + c0);
                const float4v k1 = *reinterpret_cast<const float4v*>(sKR + rr * LKR + c0 + 4);
                const float4v q0 = *reinterpret_cast<const float4v*>(sQR + rr * LKR + c0);
                const float4v q1 = *reinterpret_cast<const float4v*>(sQR + rr * LKR + c0 + 4);
                float xk[8] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
                float xq[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
                if (si >= 0) {
                    const float4v s0 = *reinterpret_cast<const float4v*>(&s_c[si][c0]);
                    const float4v s1 = *reinterpret_cast<const float4v*>(&s_c[si][c0 + 4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        xk[e] *= s0[e];
                        xq[e] *= s0[e];
                        xk[4 + e] *= s1[e];
                        xq[4 + e] *= s1[e];
                    }
                }
                Frag<OpT> Ak, Aq, Be, Bw;
                set_frag(Ak, xk);
                set_frag(Aq, xq);
                Be.load(sEH + jj * LEH + c0);
                Bw.load(sWH + jj * LEH + c0);
                mma(Ak, Be, aMe);
                mma(Ak, Bw, aMw);
                mma(Aq, Be, aAe);
                mma(Aq, Bw, aAw);
            }
            // lane: column 16J + l16, rows 16R + 4 g4 + e; a block below the
            // diagonal also clears its mirror above it
            const int j = 16 * J + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * R + 4 * g4 + e;
                const bool keepM = J < R || j < r, keepA = J < R || j <= r;
                sME[r * LM32 + j] = keepM ? aMe[e] : 0.f;
                sMW[r * LM16 + j] = from_f32<OpT>(keepM ? aMw[e] : 0.f);
                sAE[r * LM16 + j] = from_f32<OpT>(keepA ? aAe[e] : 0.f);
                sAW[r * LM16 + j] = from_f32<OpT>(keepA ? aAw[e] : 0.f);
                if (J < R) {
                    const int ru = 16 * J + 4 * g4 + e, ju = 16 * R + l16;
                    sME[ru * LM32 + ju] = 0.f;
                    sMW[ru * LM16 + ju] = from_f32<OpT>(0.f);
                    sAE[ru * LM16 + ju] = from_f32<OpT>(0.f);
                    sAW[ru * LM16 + ju] = from_f32<OpT>(0.f);
                }
            }
        }
    }
    // diagonal blocks with a decay range beyond fp16 operands:
    // 2^(G_r - G_i) = prod_{s=i+1..r} alpha_s, accumulated as a running product
    if constexpr (GATE != GATE_NONE) {
        if (flags && tid < 256) {
            constexpr int CPG = D / 16;  // channels per lane
            const int rr = tid >> 4, cg = tid & 15;
#pragma unroll 1
            for (int R = 0; R < 4; ++R) {
                if (!((flags >> R) & 1)) continue;
                const int r = 16 * R + rr;
                const bool okr = r < nvalid;
                float kr[CPG], qr[CPG], f[CPG];
#pragma unroll
                for (int m = 0; m < CPG; ++m) {
                    const int64_t e = base + (okr ? r : 0) * tokstride + cg * CPG + m;
                    kr[m] = okr ? to_f32(k[e]) : 0.f;
                    qr[m] = okr ? to_f32(q[e]) : 0.f;
                    f[m] = 1.f;
                }
#pragma unroll 1
                for (int i = 15; i >= 0; --i) {
                    const int ii = 16 * R + i;
                    float me = 0.f, mw = 0.f, ae = 0.f, aw = 0.f;
                    if (ii <= r) {
                        if (ii < r) {  // include alpha_{ii+1}
                            const int s = ii + 1;
                            const bool oks = s < nvalid;
#pragma unroll
                            for (int m = 0; m < CPG; ++m) {
                                const int64_t e = base + (oks ? s : 0) * tokstride + cg * CPG + m;
                                const float a = GATE == GATE_CHANNEL ? alpha[e] : alpha[e / D];
                                f[m] *= oks ? a : 1.f;
                            }
                        }
                        const bool oki = ii < nvalid;
#pragma unroll
                        for (int m = 0; m < CPG; ++m) {
                            const int64_t e = base + (oki ? ii : 0) * tokstride + cg * CPG + m;
                            const float ki = oki ? to_f32(k[e]) : 0.f;
                            const float ek = erase[e] * ki * f[m], wk = write[e] * ki * f[m];
                            me += kr[m] * ek;
                            mw += kr[m] * wk;
                            ae += qr[m] * ek;
                            aw += qr[m] * wk;
                        }
                    }
#pragma unroll
                    for (int off = 1; off < 16; off <<= 1) {
                        me += __shfl_xor(me, off);
                        mw += __shfl_xor(mw, off);
                        ae += __shfl_xor(ae, off);
                        aw += __shfl_xor(aw, off);
                    }
                    if (cg == 0) {
                        sME[r * LM32 + ii] = ii < r ? me : 0.f;
                        sMW[r * LM16 + ii] = from_f32<OpT>(ii < r ? mw : 0.f);
                        sAE[r * LM16 + ii] = from_f32<OpT>(ii <= r ? ae : 0.f);
                        sAW[r * LM16 + ii] = from_f32<OpT>(ii <= r ? aw : 0.f);
                    }
                }
            }
        }
    }
    __syncthreads();  // the matrices are complete; region A is free

    // ---- operands of the products below: Kt^T, V^T, Wb^T ([D][64]), Qt
#pragma unroll
    for (int j = 0; j < RPP; j += 4) {
        float4v x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = kt[j + e];
        *reinterpret_cast<float4v*>(sKTT + cc * LT32 + r0 + j) = x;
    }
#pragma unroll
    for (int j = 0; j < RPP; j += 8) {
        store_run<OpT, 8>(sVT + cc * LT16 + r0 + j, vv + j);
        store_run<OpT, 8>(sWBT + cc * LT16 + r0 + j, wb + j);
    }
#pragma unroll
    for (int j = 0; j < RPP; ++j) sQTS[frag_off<D>(r0 + j, cc)] = from_f32<OpT>(qt[j]);
    __syncthreads();

    // ---- X = Wb^T V [D][D] (accumulator order): wave's column tile nt, TX row tiles
    {
        constexpr int TX = NCT * NCT / NW;
        const int nt = wid % NCT, mt0 = (wid / NCT) * TX;
        Frag<OpT> fv[2];
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) fv[kq].load(sVT + (16 * nt + l16) * LT16 + 32 * kq + kg);
        float* X = ws.X + ch * D * D;
#pragma unroll
        for (int i = 0; i < TX; ++i) {
            const int mt = mt0 + i;
            float4v acc = zero4();
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                Frag<OpT> fw;
                fw.load(sWBT + (16 * mt + l16) * LT16 + 32 * kq + kg);
                mma(fw, fv[kq], acc);
            }
            *reinterpret_cast<float4v*>(X + ((mt * NCT + nt) * WAVE + lane) * 4) = acc;
        }
    }
    // A = A_e and Qt, fragment order, 16-byte pieces
    {
        OpT* A = static_cast<OpT*>(ws.A) + ch * CHUNK * CHUNK;
        const int r = tid / (CHUNK / 8), j0 = 8 * (tid % (CHUNK / 8));
        *reinterpret_cast<half8*>(A + frag_off<CHUNK>(r, j0)) = *reinterpret_cast<const half8*>(sAE + r * LM16 + j0);
        OpT* Qt = static_cast<OpT*>(ws.Qt) + ch * CHUNK * D;
#pragma unroll
        for (int i = tid; i < CHUNK * D / 8; i += NT2)
            *reinterpret_cast<half8*>(Qt + 8 * i) = *reinterpret_cast<const half8*>(sQTS + 8 * i);
    }
    // diagonal inverses N_RR = (I + M_e[R,R])^-1: wave R, lane j solves column j
    if (wid < 4 && lane < 16) {
        const int R = wid;
        const float* Mb = sME + (16 * R) * LM32 + 16 * R;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = r == lane ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            float m[16];
#pragma unroll
            for (int j4 = 0; j4 < (r + 3) / 4; ++j4) {
                const float4v t = *reinterpret_cast<const float4v*>(Mb + r * LM32 + 4 * j4);
#pragma unroll
                for (int e = 0; e < 4; ++e) m[4 * j4 + e] = t[e];
            }
            float acc = x[r];
#pragma unroll
            for (int j = 0; j < r; ++j) acc -= m[j] * x[j];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sN[(R * 16 + r) * LN + lane] = x[r];
    }
    __syncthreads();  // N_RR ready; Wb^T is dead (its space stages W)

    // ---- solve, M_w V and Y = A_w V, by 16-column tiles: tile t < NCT is
    // column tile t of Kt (giving W), t >= NCT column tile t - NCT of V
    // (giving Vt = N M_w V, stored as Ut = -Vt, and Y)
    {
        constexpr int TS = 2 * NCT / NW;  // tiles per wave
        float4v Z[TS][4];
#pragma unroll
        for (int s = 0; s < TS; ++s) {
            const int t = wid + NW * s;
            if (t < NCT) {
#pragma unroll
                for (int R = 0; R < 4; ++R)
                    Z[s][R] = *reinterpret_cast<const float4v*>(sKTT + (16 * t + l16) * LT32 + 16 * R + 4 * g4);
            } else {
                const int u = t - NCT;
                Frag<OpT> fv[2];
#pragma unroll
                for (int kq = 0; kq < 2; ++kq) fv[kq].load(sVT + (16 * u + l16) * LT16 + 32 * kq + kg);
                float* Y = ws.Y + ch * CHUNK * D;
#pragma unroll
                for (int R = 0; R < 4; ++R) {
                    float4v am = zero4(), ay = zero4();
#pragma unroll
                    for (int kq = 0; kq < 2; ++kq) {
                        Frag<OpT> fm, fa;
                        fm.load(sMW + (16 * R + l16) * LM16 + 32 * kq + kg);
                        fa.load(sAW + (16 * R + l16) * LM16 + 32 * kq + kg);
                        mma(fm, fv[kq], am);
                        mma(fa, fv[kq], ay);
                    }
                    Z[s][R] = am;
                    *reinterpret_cast<float4v*>(Y + ((R * NCT + u) * WAVE + lane) * 4) = ay;
                }
            }
        }
#pragma unroll
        for (int R = 0; R < 4; ++R) {
#pragma unroll
            for (int K = 0; K < R; ++K) {
                float4v m = *reinterpret_cast<const float4v*>(sME + (16 * R + l16) * LM32 + 16 * K + 4 * g4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int s = 0; s < TS; ++s)
                        Z[s][R] = __builtin_amdgcn_mfma_f32_16x16x4f32(-m[i], Z[s][K][i], Z[s][R], 0, 0, 0);
                }
            }
            const float4v n = *reinterpret_cast<const float4v*>(sN + (R * 16 + l16) * LN + 4 * g4);
#pragma unroll
            for (int s = 0; s < TS; ++s) {
                float4v z = zero4();
#pragma unroll
                for (int i = 0; i < 4; ++i) z = __builtin_amdgcn_mfma_f32_16x16x4f32(n[i], Z[s][R][i], z, 0, 0, 0);
                Z[s][R] = z;
            }
        }
        OpT* Ut = static_cast<OpT*>(ws.Ut) + ch * CHUNK * D;
#pragma unroll
        for (int s = 0; s < TS; ++s) {
            const int t = wid + NW * s;
            if (t < NCT) {
#pragma unroll
                for (int R = 0; R < 4; ++R) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sWS[frag_off<D>(16 * R + 4 * g4 + e, 16 * t + l16)] = from_f32<OpT>(Z[s][R][e]);
                }
            } else {
                const int u = t - NCT;
#pragma unroll
                for (int R = 0; R < 4; ++R) store4<OpT>(Ut + cfrag_off<D>(16 * R + 4 * g4, 16 * u + l16), -Z[s][R]);
            }
        }
    }
    __syncthreads();
    // W in fragment order, 16-byte pieces
    {
        OpT* W = static_cast<OpT*>(ws.W) + ch * CHUNK * D;
#pragma unroll
        for (int i = tid; i < CHUNK * D / 8; i += NT2)
            *reinterpret_cast<half8*>(W + 8 * i) = *reinterpret_cast<const half8*>(sWS + 8 * i);
    }
}

// One Gated DeltaNet-2 step per (sequence, head) slab, the state read once and
// written once (the structure of the KDA decode step):
//     p = S^T (alpha*k), r = S^T (alpha*q),
//     S <- Diag(alpha) S - (e*k) p^T + (w*k) v^T,
//     o = scale (r - (q.(e*k)) p + (q.(w*k)) v)   (= scale S_new^T q)
template <int D, int GATE, bool IN_F32, bool OUT_F32>
__global__ __launch_bounds__(256) void gdn2_decode_kernel(int64_t nslab, float scale, const void* __restrict__ q_,
                                                          const void* __restrict__ k_, const void* __restrict__ v_,
                                                          const float* __restrict__ erase,
                                                          const float* __restrict__ write,
                                                          const float* __restrict__ alpha, float* __restrict__ S,
                                                          void* __restrict__ o_) {
    using InT = typename InType<IN_F32>::T;
    using OutT = typename InType<OUT_F32>::T;
    constexpr int TPR = D / 4;     // threads per state row (float4 each)
    constexpr int RG = 256 / TPR;  // row groups
    constexpr int RPT = D / RG;    // rows per thread

    const int64_t slab = blockIdx.x;
    if (slab >= nslab) return;
    const int tid = threadIdx.x;
    const int rg = tid / TPR, cg = tid % TPR;
    const InT* q = reinterpret_cast<const InT*>(q_) + slab * D;
    const InT* k = reinterpret_cast<const InT*>(k_) + slab * D;
    const InT* v = reinterpret_cast<const InT*>(v_) + slab * D;
    OutT* o = reinterpret_cast<OutT*>(o_) + slab * D;
    float4v* Sv = reinterpret_cast<float4v*>(S + slab * (int64_t)D * D);

    __shared__ float s_ak[D], s_aq[D], s_ek[D], s_wk[D], s_a[D];
    __shared__ float s_p[RG][D], s_r[RG][D];
    __shared__ float s_dot[2][2];

    float4v st[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) st[m] = __builtin_nontemporal_load(&Sv[(rg + m * RG) * TPR + cg]);

    if (tid < D) {
        float a = 1.f;
        if constexpr (GATE == GATE_SCALAR) a = alpha[slab];
        if constexpr (GATE == GATE_CHANNEL) a = alpha[slab * D + tid];
        const float kk = to_f32(k[tid]), qq = to_f32(q[tid]);
        const float ek = erase[slab * D + tid] * kk, wk = write[slab * D + tid] * kk;
        s_a[tid] = a;
        s_ak[tid] = a * kk;
        s_aq[tid] = a * qq;
        s_ek[tid] = ek;
        s_wk[tid] = wk;
        float qe = qq * ek, qw = qq * wk;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            qe += __shfl_xor(qe, off);
            qw += __shfl_xor(qw, off);
        }
        if ((tid & 63) == 0) {
            s_dot[tid >> 6][0] = qe;
            s_dot[tid >> 6][1] = qw;
        }
    }
    __syncthreads();
    const float qe = D == 128 ? s_dot[0][0] + s_dot[1][0] : s_dot[0][0];
    const float qw = D == 128 ? s_dot[0][1] + s_dot[1][1] : s_dot[0][1];

    float4v p = zero4(), r = zero4();
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + m * RG;
        p += st[m] * s_ak[i];
        r += st[m] * s_aq[i];
    }
    *reinterpret_cast<float4v*>(&s_p[rg][4 * cg]) = p;
    *reinterpret_cast<float4v*>(&s_r[rg][4 * cg]) = r;
    __syncthreads();
    float4v pt = zero4(), rt = zero4();
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        pt += *reinterpret_cast<const float4v*>(&s_p[g][4 * cg]);
        rt += *reinterpret_cast<const float4v*>(&s_r[g][4 * cg]);
    }
    float vv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = to_f32(v[4 * cg + e]);
    if (rg == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[4 * cg + e] = from_f32<OutT>(scale * (rt[e] - qe * pt[e] + qw * vv[e]));
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + m * RG;
        const float a = s_a[i], ek = s_ek[i], wk = s_wk[i];
        float4v sn;
#pragma unroll
        for (int e = 0; e < 4; ++e) sn[e] = __builtin_fmaf(a, st[m][e], wk * vv[e] - ek * pt[e]);
        __builtin_nontemporal_store(sn, &Sv[i * TPR + cg]);
    }
}

template <int D, int GATE, bool IN_F32>
hipError_t intra_t(int64_t B, int64_t T, int H, int64_t NC, const void* q, const void* k, const void* v,
                   const float* erase, const float* write, const float* alpha, const ChunkWs& ws, ChunkRange cr,
                   hipStream_t stream) {
    const int64_t nch = B * H * cr.n;
    if (nch == 0) return hipSuccess;
    if constexpr (IN_F32)
        hipLaunchKernelGGL((gdn2_intra_kernel<D, GATE, true>), dim3((unsigned)nch), dim3(NT2), 0, stream, T, H, NC, q,
                           k, v, erase, write, alpha, ws, cr);
    else
        hipLaunchKernelGGL((gdn2_intra_h_kernel<D, GATE>), dim3((unsigned)nch), dim3(NT2), 0, stream, T, H, NC, q, k,
                           v, erase, write, alpha, ws, cr);
    return hipGetLastError();
}

template <int D, int GATE>
hipError_t intra_g(bool in_f32, int64_t B, int64_t T, int H, int64_t NC, const void* q, const void* k, const void* v,
                   const float* erase, const float* write, const float* alpha, const ChunkWs& ws, ChunkRange cr,
                   hipStream_t stream) {
    return in_f32 ? intra_t<D, GATE, true>(B, T, H, NC, q, k, v, erase, write, alpha, ws, cr, stream)
                  : intra_t<D, GATE, false>(B, T, H, NC, q, k, v, erase, write, alpha, ws, cr, stream);
}

template <int D>
hipError_t intra_d(int gate, bool in_f32, int64_t B, int64_t T, int H, int64_t NC, const void* q, const void* k,
                   const void* v, const float* erase, const float* write, const float* alpha, const ChunkWs& ws,
                   ChunkRange cr, hipStream_t stream) {
    if (gate == GATE_NONE)
        return intra_g<D, GATE_NONE>(in_f32, B, T, H, NC, q, k, v, erase, write, alpha, ws, cr, stream);
    if (gate == GATE_SCALAR)
        return intra_g<D, GATE_SCALAR>(in_f32, B, T, H, NC, q, k, v, erase, write, alpha, ws, cr, stream);
    return intra_g<D, GATE_CHANNEL>(in_f32, B, T, H, NC, q, k, v, erase, write, alpha, ws, cr, stream);
}

template <int D, int GATE, bool IN_F32, bool OUT_F32>
hipError_t decode_t(int64_t nslab, float scale, const void* q, const void* k, const void* v, const float* erase,
                    const float* write, const float* alpha, float* S, void* o, hipStream_t stream) {
    hipLaunchKernelGGL((gdn2_decode_kernel<D, GATE, IN_F32, OUT_F32>), dim3((unsigned)nslab), dim3(256), 0, stream,
                       nslab, scale, q, k, v, erase, write, alpha, S, o);
    return hipGetLastError();
}

template <int D, int GATE>
hipError_t decode_g(bool in_f32, bool out_f32, int64_t nslab, float scale, const void* q, const void* k,
                    const void* v, const float* erase, const float* write, const float* alpha, float* S, void* o,
                    hipStream_t stream) {
    if (in_f32)
        return out_f32 ? decode_t<D, GATE, true, true>(nslab, scale, q, k, v, erase, write, alpha, S, o, stream)
                       : decode_t<D, GATE, true, false>(nslab, scale, q, k, v, erase, write, alpha, S, o, stream);
    return out_f32 ? decode_t<D, GATE, false, true>(nslab, scale, q, k, v, erase, write, alpha, S, o, stream)
                   : decode_t<D, GATE, false, false>(nslab, scale, q, k, v, erase, write, alpha, S, o, stream);
}

template <int D>
hipError_t decode_d(int gate, bool in_f32, bool out_f32, int64_t nslab, float scale, const void* q, const void* k,
                    const void* v, const float* erase, const float* write, const float* alpha, float* S, void* o,
                    hipStream_t stream) {
    if (gate == GATE_NONE)
        return decode_g<D, GATE_NONE>(in_f32, out_f32, nslab, scale, q, k, v, erase, write, alpha, S, o, stream);
    if (gate == GATE_SCALAR)
        return decode_g<D, GATE_SCALAR>(in_f32, out_f32, nslab, scale, q, k, v, erase, write, alpha, S, o, stream);
    return decode_g<D, GATE_CHANNEL>(in_f32, out_f32, nslab, scale, q, k, v, erase, write, alpha, S, o, stream);
}

}  // namespace

hipError_t launch_gdn2_intra(int D, int gate, bool in_f32, int64_t B, int64_t T, int H, int64_t NC, const void* q,
                             const void* k, const void* v, const float* erase, const float* write,
                             const float* alpha, const ChunkWs& ws, ChunkRange cr, hipStream_t stream) {
    if (D == 64) return intra_d<64>(gate, in_f32, B, T, H, NC, q, k, v, erase, write, alpha, ws, cr, stream);
    return intra_d<128>(gate, in_f32, B, T, H, NC, q, k, v, erase, write, alpha, ws, cr, stream);
}

hipError_t launch_gdn2_decode(int D, int gate, bool in_f32, bool out_f32, int64_t nslab, float scale, const void* q,
                              const void* k, const void* v, const float* erase, const float* write,
                              const float* alpha, float* S, void* o, hipStream_t stream) {
    if (nslab == 0) return hipSuccess;
    if (D == 64) return decode_d<64>(gate, in_f32, out_f32, nslab, scale, q, k, v, erase, write, alpha, S, o, stream);
    return decode_d<128>(gate, in_f32, out_f32, nslab, scale, q, k, v, erase, write, alpha, S, o, stream);
}

}  // namespace gdr
