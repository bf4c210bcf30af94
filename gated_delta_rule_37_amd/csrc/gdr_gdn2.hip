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
// Range of the decay factors: every product of a row factor 2^(G_r - ref) and a
// column factor 2^(ref - G_j) uses a reference between the two (the end of the
// column block for blocks below the diagonal, so both factors are at most 1;
// the start of the block on the diagonal, where the column factor is at most
// 2^rho for the block's decay range rho).  A diagonal block whose range exceeds
// 60 (in log2) is computed pair by pair with 2^(G_r - G_j) formed directly.
// The four C x C matrices are formed with fp32 operands on matrix cores.  For
// bf16 inputs the three products with V (X, Y, M_w V) take fp16 operands and
// the pass's operands W, Ut, Qt, KbT, A are stored in fp16 (the operand
// precision of the KDA path); X and Y stay fp32.  fp32 inputs keep fp32 throughout.
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

template <int D, int GATE, bool IN_F32>
__global__ __launch_bounds__(NT2) void gdn2_intra_kernel(int64_t T, int H, int64_t NC, const void* __restrict__ q_,
                                                         const void* __restrict__ k_, const void* __restrict__ v_,
                                                         const float* __restrict__ erase,
                                                         const float* __restrict__ write,
                                                         const float* __restrict__ alpha, ChunkWs ws) {
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

    const int64_t ch = blockIdx.x;  // chunk-head: (b * H + h) * NC + c
    const int64_t bh = ch / NC, c = ch % NC;
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
                   const float* erase, const float* write, const float* alpha, const ChunkWs& ws,
                   hipStream_t stream) {
    const int64_t nch = B * H * NC;
    if (nch == 0) return hipSuccess;
    hipLaunchKernelGGL((gdn2_intra_kernel<D, GATE, IN_F32>), dim3((unsigned)nch), dim3(NT2), 0, stream, T, H, NC, q,
                       k, v, erase, write, alpha, ws);
    return hipGetLastError();
}

template <int D, int GATE>
hipError_t intra_g(bool in_f32, int64_t B, int64_t T, int H, int64_t NC, const void* q, const void* k, const void* v,
                   const float* erase, const float* write, const float* alpha, const ChunkWs& ws,
                   hipStream_t stream) {
    return in_f32 ? intra_t<D, GATE, true>(B, T, H, NC, q, k, v, erase, write, alpha, ws, stream)
                  : intra_t<D, GATE, false>(B, T, H, NC, q, k, v, erase, write, alpha, ws, stream);
}

template <int D>
hipError_t intra_d(int gate, bool in_f32, int64_t B, int64_t T, int H, int64_t NC, const void* q, const void* k,
                   const void* v, const float* erase, const float* write, const float* alpha, const ChunkWs& ws,
                   hipStream_t stream) {
    if (gate == GATE_NONE) return intra_g<D, GATE_NONE>(in_f32, B, T, H, NC, q, k, v, erase, write, alpha, ws, stream);
    if (gate == GATE_SCALAR)
        return intra_g<D, GATE_SCALAR>(in_f32, B, T, H, NC, q, k, v, erase, write, alpha, ws, stream);
    return intra_g<D, GATE_CHANNEL>(in_f32, B, T, H, NC, q, k, v, erase, write, alpha, ws, stream);
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
                             const float* alpha, const ChunkWs& ws, hipStream_t stream) {
    if (D == 64) return intra_d<64>(gate, in_f32, B, T, H, NC, q, k, v, erase, write, alpha, ws, stream);
    return intra_d<128>(gate, in_f32, B, T, H, NC, q, k, v, erase, write, alpha, ws, stream);
}

hipError_t launch_gdn2_decode(int D, int gate, bool in_f32, bool out_f32, int64_t nslab, float scale, const void* q,
                              const void* k, const void* v, const float* erase, const float* write,
                              const float* alpha, float* S, void* o, hipStream_t stream) {
    if (nslab == 0) return hipSuccess;
    if (D == 64) return decode_d<64>(gate, in_f32, out_f32, nslab, scale, q, k, v, erase, write, alpha, S, o, stream);
    return decode_d<128>(gate, in_f32, out_f32, nslab, scale, q, k, v, erase, write, alpha, S, o, stream);
}

}  // namespace gdr
