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

// Operand fragments of one chunk, held in registers exactly as loaded (no
// conversion at load time, so issuing a prefetch never waits for it).
// XY: the chunk also carries the additive terms of the separate-gate variant
// (Gated DeltaNet-2): x, this lane's part of the state term X added after the
// chunk's update, and y, its part of the output term Y (fp32, accumulator order).
template <int D, bool IN_F32, bool XY = false>
struct ChunkFrags {
    using OpT = typename StateCfg<D, IN_F32>::OpT;
    static constexpr int SRT = StateCfg<D, IN_F32>::SRT;
    Frag<OpT> w[D / 32], q[D / 32], a[2], kb[SRT][2];
    OpT ut[4];
    float gam[SRT][4];
    float x[XY ? SRT : 1][4], y[4];
};

// All chunk operands are stored in fragment order by the intra-chunk kernel:
// every fragment below is one contiguous, fully coalesced 1 KiB (fp16) load.
template <int D, bool IN_F32, bool XY = false>
__device__ __forceinline__ void load_chunk(ChunkFrags<D, IN_F32, XY>& f, const ChunkWs& ws, int64_t ch,
                                           int j0, int wid, int lane) {
    using Cfg = StateCfg<D, IN_F32>;
    using OpT = typename Cfg::OpT;
    const OpT* W = reinterpret_cast<const OpT*>(ws.W) + ch * CHUNK * D + (wid * (D / 32) * 64 + lane) * 8;
    const OpT* Q = reinterpret_cast<const OpT*>(ws.Qt) + ch * CHUNK * D + (wid * (D / 32) * 64 + lane) * 8;
#pragma unroll
    for (int kq = 0; kq < D / 32; ++kq) {
        f.w[kq].load(W + kq * 64 * 8);
        f.q[kq].load(Q + kq * 64 * 8);
    }
    const OpT* A = reinterpret_cast<const OpT*>(ws.A) + ch * CHUNK * CHUNK + (wid * 2 * 64 + lane) * 8;
    f.a[0].load(A);
    f.a[1].load(A + 64 * 8);  // zero for waves 0 and 1 (A is lower triangular)
    const OpT* KbT = reinterpret_cast<const OpT*>(ws.KbT) + ch * D * CHUNK;
#pragma unroll
    for (int m = 0; m < Cfg::SRT; ++m) {
        const int rt = wid * (D / 64) + m;  // 16-row tile of the state
        f.kb[m][0].load(KbT + ((rt * 2 + 0) * 64 + lane) * 8);
        f.kb[m][1].load(KbT + ((rt * 2 + 1) * 64 + lane) * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) f.gam[m][e] = ws.gam[ch * D + 16 * rt + 4 * (lane >> 4) + e];
    }
    // Ut in accumulator order: this lane's four rows of its column
    const OpT* Ut = reinterpret_cast<const OpT*>(ws.Ut) + ch * CHUNK * D + ((wid * (D / 16) + j0 / 16) * 64 + lane) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) f.ut[e] = Ut[e];
    if constexpr (XY) {
        // X [D][D] and Y [64][D], accumulator order: this lane's four rows of
        // column j0 + lane % 16 of the wave's state tiles and output rows
#pragma unroll
        for (int m = 0; m < Cfg::SRT; ++m) {
            const int rt = wid * (D / 64) + m;
            const float4v xv = *reinterpret_cast<const float4v*>(
                ws.X + ch * D * D + ((rt * (D / 16) + j0 / 16) * 64 + lane) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) f.x[m][e] = xv[e];
        }
        const float4v yv = *reinterpret_cast<const float4v*>(
            ws.Y + ch * CHUNK * D + ((wid * (D / 16) + j0 / 16) * 64 + lane) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) f.y[e] = yv[e];
    }
}

template <typename OpT>
__device__ __forceinline__ void store8(OpT* dst, const OpT (&v)[8]) {
    if constexpr (sizeof(OpT) == 2) {
        half8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = v[e];
        *reinterpret_cast<half8*>(dst) = h;
    } else {
        float4v a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = v[e];
            b[e] = v[4 + e];
        }
        reinterpret_cast<float4v*>(dst)[0] = a;
        reinterpret_cast<float4v*>(dst)[1] = b;
    }
}

template <typename OpT>
__device__ __forceinline__ void st4(OpT* dst, const float4v& v) {
    if constexpr (sizeof(OpT) == 2) {
        half4 h;
        h[0] = from_f32<_Float16>(v[0]); h[1] = from_f32<_Float16>(v[1]);
        h[2] = from_f32<_Float16>(v[2]); h[3] = from_f32<_Float16>(v[3]);
        *reinterpret_cast<half4*>(dst) = h;
    } else {
        *reinterpret_cast<float4v*>(dst) = v;
    }
}

template <int D, bool IN_F32, bool OUT_F32, bool SAVE, bool HAS_O, bool XY = false>
__device__ __forceinline__ void state_step(const ChunkFrags<D, IN_F32, XY>& cur, int64_t c, int64_t T, int H,
                                           int64_t b, int h, int64_t bh, int64_t NC, int j0, int wid,
                                           int l16, int g4, float scale, const ChunkWs& ws,
                                           float4v (&S)[StateCfg<D, IN_F32>::SRT],
                                           typename StateCfg<D, IN_F32>::OpT* s_S,
                                           typename StateCfg<D, IN_F32>::OpT* s_U,
                                           typename InType<OUT_F32>::T* o) {
    using Cfg = StateCfg<D, IN_F32>;
    using OpT = typename Cfg::OpT;
    using OutT = typename InType<OUT_F32>::T;
    constexpr int SRT = Cfg::SRT, LDS_S = Cfg::LDS_S, LDS_U = Cfg::LDS_U;
    const int64_t ch = bh * NC + c;

    // U = Ut - W S and the inter-chunk part of the output, O = Qt S
    float4v u = zero4(), oacc = zero4();
#pragma unroll
    for (int kq = 0; kq < D / 32; ++kq) {
        Frag<OpT> fs;
        fs.load(s_S + l16 * LDS_S + 32 * kq + 8 * g4);
        mma(cur.w[kq], fs, u);
        if constexpr (HAS_O) mma(cur.q[kq], fs, oacc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = to_f32(cur.ut[e]) - u[e];
    st4<OpT>(s_U + l16 * LDS_U + 16 * wid + 4 * g4, u);
    __syncthreads();
    if constexpr (SAVE) {
        // U of this chunk, fragment order (rows position, k = value column):
        // waves 0 and 1, each 16-lane group 16 positions and 8 of the columns
        if (wid < 2) {
            const int grp = 4 * wid + g4, pos0 = 16 * (grp & 3), hf = grp >> 2;
            OpT vals[8];
            lds_column8<LDS_U>(s_U, 8 * hf, pos0, l16, vals);
            store8(reinterpret_cast<OpT*>(ws.Usave) + ch * CHUNK * D + frag_off<D>(pos0 + l16, j0 + 8 * hf), vals);
        }
    }

    Frag<OpT> fu0, fu1;
    fu0.load(s_U + l16 * LDS_U + 8 * g4);
    fu1.load(s_U + l16 * LDS_U + 32 + 8 * g4);
    // intra-chunk part of the output, O += A U
    if constexpr (HAS_O) {
        mma(cur.a[0], fu0, oacc);
        mma(cur.a[1], fu1, oacc);  // zero block for waves 0 and 1
        if constexpr (XY) {
#pragma unroll
            for (int e = 0; e < 4; ++e) oacc[e] += cur.y[e];
        }
        const int64_t tbase = c * CHUNK + 16 * wid + 4 * g4;
        OutT* op = o + ((b * T + tbase) * H + h) * D + j0 + l16;
        const int64_t tstride = static_cast<int64_t>(H) * D;
        if (tbase + 3 < T) {
#pragma unroll
            for (int e = 0; e < 4; ++e) op[e * tstride] = from_f32<OutT>(scale * oacc[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (tbase + e < T) op[e * tstride] = from_f32<OutT>(scale * oacc[e]);
        }
    }

    if constexpr (SAVE) {
        // chunk-start state snapshot [D][D] in operand precision, fragment order
        // (rows d, k = value column): eight consecutive columns per lane, read
        // as columns of the transposed LDS copy.  Each wave saves the rows it
        // owns (each 16-lane group 16 rows and 8 of the columns), which no
        // other wave writes, before it overwrites them below.
        constexpr int RW = D / 4, RG = RW / 16;
        if (g4 < 2 * RG) {
            const int d0 = RW * wid + 16 * (g4 % RG), hf = g4 / RG;
            OpT vals[8];
            lds_column8<LDS_S>(s_S, 8 * hf, d0, l16, vals);
            store8(reinterpret_cast<OpT*>(ws.Ssnap) + ch * D * D + frag_off<D>(d0 + l16, j0 + 8 * hf), vals);
        }
    }

    // S <- Diag(gamma) S + Kb^T U
#pragma unroll
    for (int m = 0; m < SRT; ++m) {
#pragma unroll
        for (int e = 0; e < 4; ++e) S[m][e] *= cur.gam[m][e];
        mma(cur.kb[m][0], fu0, S[m]);
        mma(cur.kb[m][1], fu1, S[m]);
        if constexpr (XY) {
#pragma unroll
            for (int e = 0; e < 4; ++e) S[m][e] += cur.x[m][e];
        }
        st4<OpT>(s_S + l16 * LDS_S + wid * (D / 4) + 16 * m + 4 * g4, S[m]);
    }
    __syncthreads();
}

// L2 warm-up for a chunk-head's operands: the eight workgroups of one head
// (one per dv slice, all on one XCD) each touch their 1/NSL share of every
// per-chunk array with one dword per 128-byte line.  Returns the loaded dwords
// XOR-ed together; the caller keeps the value alive so the loads are issued.
template <int D, bool IN_F32>
struct L2Touch {
    using OpT = typename StateCfg<D, IN_F32>::OpT;
    static constexpr int NSL = StateCfg<D, IN_F32>::NSL;
    static constexpr int LINE = 128;
    static constexpr int QL = CHUNK * D * (int)sizeof(OpT) / NSL / LINE;      // lines per slice, [64][D]
    static constexpr int AL = CHUNK * CHUNK * (int)sizeof(OpT) / NSL / LINE;  // lines per slice, A
    static constexpr int GL = (D * 4 + LINE - 1) / LINE;                      // gamma lines (slice 0)
    static constexpr int NL = 4 * QL + AL + GL;
    static constexpr int NPF = (NL + WAVE - 1) / WAVE;  // loads per lane per chunk
};

template <int D, bool IN_F32, int NPF>
__device__ __forceinline__ void touch_chunk(uint32_t (&out)[NPF], const ChunkWs& ws, int64_t ch, int slice,
                                            int lane) {
    using P = L2Touch<D, IN_F32>;
    using OpT = typename P::OpT;
    const size_t mat = size_t(CHUNK) * D * sizeof(OpT);
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
        const int L = lane + WAVE * i;
        const char* addr;
        const int reg = L / P::QL;
        if (L < 4 * P::QL) {
            const char* base = reg == 0   ? static_cast<const char*>(ws.W)
                               : reg == 1 ? static_cast<const char*>(ws.Qt)
                               : reg == 2 ? static_cast<const char*>(ws.KbT)
                                          : static_cast<const char*>(ws.Ut);
            addr = base + ch * mat + size_t(slice * P::QL + L % P::QL) * P::LINE;
        } else if (L < 4 * P::QL + P::AL) {
            addr = static_cast<const char*>(ws.A) + ch * size_t(CHUNK) * CHUNK * sizeof(OpT) +
                   size_t(slice * P::AL + (L - 4 * P::QL)) * P::LINE;
        } else {
            // gamma: slice 0 only; other slices re-touch their first W line
            const int gl = L - 4 * P::QL - P::AL;
            addr = (slice == 0 && gl < P::GL)
                       ? reinterpret_cast<const char*>(ws.gam + ch * D) + size_t(gl) * P::LINE
                       : static_cast<const char*>(ws.W) + ch * mat + size_t(slice * P::QL) * P::LINE;
        }
        out[i] = *reinterpret_cast<const uint32_t*>(addr);
    }
}

template <int D, bool IN_F32, bool OUT_F32, bool SAVE, bool HAS_O, bool XY = false>
__global__ __launch_bounds__(320) void state_fwd_kernel(int64_t T, int H, int64_t NC, float scale,
                                                        ChunkWs ws, const float* S0,
                                                        float* ST, void* __restrict__ o_, ChunkRange cr) {
    // Chunks cr.lo .. cr.lo + cr.n - 1 of every (batch, head); the state enters
    // from S0 (NULL: zero) and leaves into ST.  S0 and ST may alias: each
    // workgroup reads its slice of S0 before it writes the same slice of ST, and
    // slices of different workgroups are disjoint.
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
    OutT* o = reinterpret_cast<OutT*>(o_);  // NULL: state pass only (backward recompute)

    // Waves 0-3 run the state pass.  Wave 4 only warms the L2 with the operands
    // of chunk c + PF while chunk c computes; it takes part in every barrier.
    if (wid == 4) {
        constexpr int PF = 8;
        constexpr int NPF = L2Touch<D, IN_F32>::NPF;
        const int slice = j0 / Cfg::NS;
        const int64_t lo = cr.lo, hi = cr.lo + cr.n;
        uint32_t ring[PF][NPF];
        uint32_t acc = 0;
        // (an empty range touches nothing: its workspace may be empty)
        if (cr.n > 0) {
#pragma unroll
            for (int s2 = 0; s2 < PF; ++s2)
                touch_chunk<D, IN_F32, NPF>(ring[s2], ws, bh * NC + (lo + s2 < NC ? lo + s2 : lo), slice, lane);
        }
        __syncthreads();
#pragma unroll 1
        for (int64_t c0 = lo; c0 < hi; c0 += PF) {
#pragma unroll
            for (int s2 = 0; s2 < PF; ++s2) {
                const int64_t c = c0 + s2;
                if (c < hi) {
#pragma unroll
                    for (int i = 0; i < NPF; ++i) acc ^= ring[s2][i];  // chunk c is in L2 by now
                    // unconditional (clamped) so every slot is refilled: no register copies
                    touch_chunk<D, IN_F32, NPF>(ring[s2], ws, bh * NC + (c + PF < NC ? c + PF : NC - 1), slice, lane);
                    __syncthreads();
                    __syncthreads();
                }
            }
        }
        asm volatile("" ::"v"(acc));
        return;
    }

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

    // Chunks are processed in pairs with two register sets used alternately,
    // so the prefetch of chunk c+1 never has to be copied into place.
    // The prefetch is unconditional (the chunk index is clamped to the last
    // chunk) so that the compiler can count outstanding loads exactly and wait
    // only for the chunk about to be used.
    ChunkFrags<D, IN_F32, XY> fa, fb;
    const int64_t lo = cr.lo, hi = cr.lo + cr.n, last = hi - 1;
    if (cr.n > 0) load_chunk<D, IN_F32, XY>(fa, ws, bh * NC + lo, j0, wid, lane);
#pragma unroll 1
    for (int64_t c = lo; c < hi; c += 2) {
        load_chunk<D, IN_F32, XY>(fb, ws, bh * NC + (c + 1 < hi ? c + 1 : last), j0, wid, lane);
        state_step<D, IN_F32, OUT_F32, SAVE, HAS_O, XY>(fa, c, T, H, b, h, bh, NC, j0, wid, l16, g4, scale, ws,
                                                        S, s_S, s_U, o);
        if (c + 1 >= hi) break;
        load_chunk<D, IN_F32, XY>(fa, ws, bh * NC + (c + 2 < hi ? c + 2 : last), j0, wid, lane);
        state_step<D, IN_F32, OUT_F32, SAVE, HAS_O, XY>(fb, c + 1, T, H, b, h, bh, NC, j0, wid, l16, g4, scale,
                                                        ws, S, s_S, s_U, o);
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

// ---------------------------------------------------------------------------
// Chain-only pass for fp16 operands, staged through LDS.
//
// Only U = Ut - W S and S <- Diag(gamma) S + Kb^T U are sequential; the output
// O = Qt S + A U is computed afterwards for all chunks in parallel from the
// saved chunk-start states and U (output_kernel).  Every step needs all of W
// and Kb^T of its chunk in each slice's CU, so the step is bounded by how fast
// a CU can take them in.  Wave 4 copies chunk c+2 from global memory straight
// into one of three LDS buffers (global_load_lds: no registers, no waits in
// the compute waves) and pulls chunk c+PF into the L2; waves 0-3 compute chunk
// c from its buffer with conflict-free 16-byte LDS reads.
// ---------------------------------------------------------------------------

template <int D, int NSW>
struct ChainStage {
    static constexpr int MAT = CHUNK * D * 2;  // [64][D] fp16
    static constexpr int W = 0;
    static constexpr int KBT = MAT;
    static constexpr int UT = 2 * MAT;          // per slice, its four 16x16 tiles of Ut (2 KiB)
    static constexpr int GAM = UT + 2048 * NSW; // D fp32 in a 1 KiB slot
    static constexpr int BYTES = GAM + 1024;
    static constexpr int ND0 = MAT / 2048 + 2 * NSW + 1;  // copies per chunk of loader wave 0
    static constexpr int NDP = MAT / 2048;                // copies per chunk of loader waves 1-3
    static constexpr int NWH = D / 16 / NSW;              // workgroups per head
    static constexpr int QL = MAT / NWH / 128;            // 128-byte lines per workgroup of one array
    static constexpr int NT = (3 * QL + 1 + 63) / 64;     // touch copies per chunk
};

// Chunk ch's operands for the NSW slices of workgroup `member` of its head
// (slices member*NSW ..) into `dst`, in four parts, one per loader wave: PART 0
// the first half of W, the slices' Ut tiles and gamma; PART 1 the second half
// of W; PARTs 2 and 3 the halves of Kb^T.
template <int D, int NSW, int PART>
__device__ __forceinline__ void stage_chain(lds_char* dst, const ChunkWs& ws, int64_t ch, int member, int lane) {
    using L = ChainStage<D, NSW>;
    constexpr int HALF = L::MAT / 2;
    if constexpr (PART == 1) {
        copy_block_to_lds<HALF / 1024>(static_cast<const char*>(ws.W) + ch * L::MAT + HALF, dst + L::W + HALF, lane);
    } else if constexpr (PART == 2) {
        copy_block_to_lds<HALF / 1024>(static_cast<const char*>(ws.KbT) + ch * L::MAT, dst + L::KBT, lane);
    } else if constexpr (PART == 3) {
        copy_block_to_lds<HALF / 1024>(static_cast<const char*>(ws.KbT) + ch * L::MAT + HALF, dst + L::KBT + HALF,
                                       lane);
    } else {
        copy_block_to_lds<HALF / 1024>(static_cast<const char*>(ws.W) + ch * L::MAT, dst + L::W, lane);
        // Ut tiles (rt, slice), rt = 0..3, 512 bytes each: two tiles per copy
        const char* U = static_cast<const char*>(ws.Ut) + ch * L::MAT;
#pragma unroll
        for (int sl = 0; sl < NSW; ++sl)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int rt = 2 * i + (lane >> 5);
                copy16_to_lds(U + (rt * (D / 16) + member * NSW + sl) * 512 + (lane & 31) * 16,
                              dst + L::UT + sl * 2048 + i * 1024);
            }
        // gamma: D floats; lanes past the end re-read the first piece into the slot's tail
        const char* G = reinterpret_cast<const char*>(ws.gam + ch * D);
        copy16_to_lds(G + (lane < D / 4 ? lane : 0) * 16, dst + L::GAM);
    }
}

template <int D, int NSW>
__device__ __forceinline__ void stage_chain_part(int part, lds_char* dst, const ChunkWs& ws, int64_t ch, int member,
                                                 int lane) {
    if (part == 0) stage_chain<D, NSW, 0>(dst, ws, ch, member, lane);
    else if (part == 1) stage_chain<D, NSW, 1>(dst, ws, ch, member, lane);
    else if (part == 2) stage_chain<D, NSW, 2>(dst, ws, ch, member, lane);
    else stage_chain<D, NSW, 3>(dst, ws, ch, member, lane);
}

// One dword of each 128-byte line of this workgroup's share of chunk ch.
template <int D, int NSW>
__device__ __forceinline__ void touch_chain(lds_char* dummy, const ChunkWs& ws, int64_t ch, int slice, int lane) {
    using L = ChainStage<D, NSW>;
    constexpr int QL = L::QL;
#pragma unroll
    for (int i = 0; i < L::NT; ++i) {
        const int Lr = lane + 64 * i;
        const char* addr;
        if (Lr < QL) addr = static_cast<const char*>(ws.W) + ch * L::MAT + (slice * QL + Lr) * 128;
        else if (Lr < 2 * QL) addr = static_cast<const char*>(ws.KbT) + ch * L::MAT + (slice * QL + Lr - QL) * 128;
        else if (Lr < 3 * QL) addr = static_cast<const char*>(ws.Ut) + ch * L::MAT + (slice * QL + Lr - 2 * QL) * 128;
        else addr = reinterpret_cast<const char*>(ws.gam + ch * D) + (slice % (D * 4 / 128)) * 128;
        copy4_to_lds(addr, dummy + i * 256);
    }
}

template <int D, int NSW>
__device__ __forceinline__ void chain_frags(ChunkFrags<D, false>& f, const lds_char* src, int sl, int wid, int lane) {
    using L = ChainStage<D, NSW>;
    constexpr int SRT = StateCfg<D, false>::SRT;
#pragma unroll
    for (int kq = 0; kq < D / 32; ++kq)
        f.w[kq].v = *reinterpret_cast<const __attribute__((address_space(3))) half8*>(src + L::W + ((wid * (D / 32) + kq) * 64 + lane) * 16);
#pragma unroll
    for (int m = 0; m < SRT; ++m) {
        const int rt = wid * (D / 64) + m;
        f.kb[m][0].v = *reinterpret_cast<const __attribute__((address_space(3))) half8*>(src + L::KBT + ((rt * 2 + 0) * 64 + lane) * 16);
        f.kb[m][1].v = *reinterpret_cast<const __attribute__((address_space(3))) half8*>(src + L::KBT + ((rt * 2 + 1) * 64 + lane) * 16);
        const float4v g = *reinterpret_cast<const __attribute__((address_space(3))) float4v*>(src + L::GAM + (16 * rt + 4 * (lane >> 4)) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) f.gam[m][e] = g[e];
    }
    const half4 u = *reinterpret_cast<const __attribute__((address_space(3))) half4*>(src + L::UT + sl * 2048 + (wid * 256 + lane * 4) * 2);
#pragma unroll
    for (int e = 0; e < 4; ++e) f.ut[e] = u[e];
}

// Waits until at most n copies of this wave are outstanding; n is one of
// 0, NT, 2NT, ND, ND+NT, ND+2NT (chosen at run time, immediates at compile time).
template <int ND, int NT>
__device__ __forceinline__ void wait_outstanding(int n) {
    if (n >= ND + 2 * NT) wait_vmcnt<ND + 2 * NT>();
    else if (n >= ND + NT) wait_vmcnt<ND + NT>();
    else if (n >= ND) wait_vmcnt<ND>();
    else if (n >= 2 * NT) wait_vmcnt<2 * NT>();
    else if (n >= NT) wait_vmcnt<NT>();
    else wait_vmcnt<0>();
}

// NSW slices per workgroup: 4*NSW compute waves (four per slice, slice sl =
// wave / 4) and four loader waves that stage each chunk's W, Kb^T and gamma once
// for all of them.  With two slices a head's state pass holds half as many CUs,
// which the intra-chunk kernels running beside it use.
template <int D, int NSW>
__global__ __launch_bounds__(64 * (4 * NSW + 4)) void state_chain_kernel(int64_t T, int H, int64_t NC, ChunkWs ws,
                                                                         const float* S0, float* ST, ChunkRange cr) {
    using Cfg = StateCfg<D, false>;
    using OpT = _Float16;
    using L = ChainStage<D, NSW>;
    constexpr int SRT = Cfg::SRT, LDS_S = Cfg::LDS_S;
    constexpr int PF = 8;

    __shared__ __attribute__((aligned(16))) OpT s_S[NSW][Cfg::NS * LDS_S];
    __shared__ __attribute__((aligned(16))) OpT s_U[NSW][Cfg::NS * Cfg::LDS_U];
    __shared__ __attribute__((aligned(1024))) char stage[3][L::BYTES];
    __shared__ __attribute__((aligned(16))) char dummy[L::NT * 256];

    const int64_t nblk = gridDim.x;
    int64_t lid = blockIdx.x;
    if (nblk % 8 == 0) lid = (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
    const int64_t bh = lid / L::NWH;
    const int member = static_cast<int>(lid % L::NWH);
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh % H);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    lds_char* const sbuf = (lds_char*)&stage[0][0];
    lds_char* const sdummy = (lds_char*)&dummy[0];
    const int64_t lo = cr.lo, hi = cr.lo + cr.n;  // chunks lo .. hi-1 (the state enters at lo)

    if (wave >= 4 * NSW) {
        // Loaders (the last four waves, one part each).  Two barriers per step,
        // like the compute waves; they never fence, so their copies stay in
        // flight across the first one.  The first loader also warms the L2
        // (also past the range: the next range's first chunks).
        const int part = wave - 4 * NSW;
        const bool w4 = part == 0;
        if (cr.n > 0) stage_chain_part<D, NSW>(part, sbuf, ws, bh * NC + lo, member, lane);
        if (cr.n > 1) stage_chain_part<D, NSW>(part, sbuf + L::BYTES, ws, bh * NC + lo + 1, member, lane);
        if (w4) {
#pragma unroll 1
            for (int64_t c = lo + 2; c < lo + PF && c < NC; ++c)
                touch_chain<D, NSW>(sdummy, ws, bh * NC + c, member, lane);
        }
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        int nb = 2;  // buffer of chunk c + 2
#pragma unroll 1
        for (int64_t c = lo; c < hi; ++c) {
            const bool st2 = c + 2 < hi, tpf = w4 && c + PF < NC;
            if (st2) stage_chain_part<D, NSW>(part, sbuf + nb * L::BYTES, ws, bh * NC + c + 2, member, lane);
            if (tpf) touch_chain<D, NSW>(sdummy, ws, bh * NC + c + PF, member, lane);
            nb = nb == 2 ? 0 : nb + 1;
            __builtin_amdgcn_s_barrier();
            // this wave's copies of chunk c+1 must have landed; later ones may stay in flight
            if (w4) {
                // the previous step's touches (issued iff it ran and touched), then this step's copies and touches
                const int n = ((c >= lo + 1 && c - 1 + PF < NC) ? L::NT : 0) + (st2 ? L::ND0 : 0) + (tpf ? L::NT : 0);
                wait_outstanding<L::ND0, L::NT>(n);
            } else if (st2) {
                wait_vmcnt<L::NDP>();
            } else {
                wait_vmcnt<0>();
            }
            __builtin_amdgcn_s_barrier();
        }
        return;
    }

    const int sl = wave >> 2, wid = wave & 3;
    const int j0 = (member * NSW + sl) * Cfg::NS;
    OpT* const sS = &s_S[sl][0];
    OpT* const sU = &s_U[sl][0];
    float4v S[SRT];
#pragma unroll
    for (int m = 0; m < SRT; ++m) {
        const int d0 = wid * (D / 4) + 16 * m + 4 * g4;
#pragma unroll
        for (int e = 0; e < 4; ++e) S[m][e] = S0 ? S0[(bh * D + d0 + e) * D + j0 + l16] : 0.f;
        st4<OpT>(sS + l16 * LDS_S + d0, S[m]);
    }
    __syncthreads();

    int cb = 0;  // buffer of chunk c
#pragma unroll 1
    for (int64_t c = lo; c < hi; ++c) {
        ChunkFrags<D, false> f;
        chain_frags<D, NSW>(f, sbuf + cb * L::BYTES, sl, wid, lane);
        cb = cb == 2 ? 0 : cb + 1;
        state_step<D, false, false, true, false>(f, c, T, H, b, h, bh, NC, j0, wid, l16, g4, 1.f, ws, S, sS, sU,
                                                 nullptr);
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
                                 bool wide, ChunkRange cr, hipStream_t stream) {
    const int64_t nblk = B * H * StateCfg<D, IN_F32>::NSL;
    if (nblk == 0) return hipSuccess;
    if constexpr (!IN_F32) {
        // fp16 operands: the chain pass always saves the chunk-start states and U;
        // the output is produced by output_kernel
        if (wide)
            hipLaunchKernelGGL((state_chain_kernel<D, 2>), dim3((unsigned)(nblk / 2)), dim3(768), 0, stream, T, H,
                               NC, ws, S0, ST, cr);
        else
            hipLaunchKernelGGL((state_chain_kernel<D, 1>), dim3((unsigned)nblk), dim3(512), 0, stream, T, H, NC,
                               ws, S0, ST, cr);
        return hipGetLastError();
    }
    if (save && o)
        hipLaunchKernelGGL((state_fwd_kernel<D, IN_F32, OUT_F32, true, true>), dim3((unsigned)nblk), dim3(320),
                           0, stream, T, H, NC, scale, ws, S0, ST, o, cr);
    else if (save)
        hipLaunchKernelGGL((state_fwd_kernel<D, IN_F32, OUT_F32, true, false>), dim3((unsigned)nblk), dim3(320),
                           0, stream, T, H, NC, scale, ws, S0, ST, o, cr);
    else
        hipLaunchKernelGGL((state_fwd_kernel<D, IN_F32, OUT_F32, false, true>), dim3((unsigned)nblk), dim3(320),
                           0, stream, T, H, NC, scale, ws, S0, ST, o, cr);
    return hipGetLastError();
}

// The separate-gate variant's pass: the register-prefetch pass with the output
// computed in it, plus the per-chunk terms X (state) and Y (output) of ws.
template <int D, bool IN_F32, bool OUT_F32>
static hipError_t launch_state_xy_t(int64_t B, int64_t T, int H, int64_t NC, float scale, const ChunkWs& ws,
                                    const float* S0, float* ST, void* o, ChunkRange cr, hipStream_t stream) {
    const int64_t nblk = B * H * StateCfg<D, IN_F32>::NSL;
    if (nblk == 0) return hipSuccess;
    hipLaunchKernelGGL((state_fwd_kernel<D, IN_F32, OUT_F32, false, true, true>), dim3((unsigned)nblk), dim3(320),
                       0, stream, T, H, NC, scale, ws, S0, ST, o, cr);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_state_xy_d(bool in_f32, bool out_f32, int64_t B, int64_t T, int H, int64_t NC, float scale,
                                    const ChunkWs& ws, const float* S0, float* ST, void* o, ChunkRange cr,
                                    hipStream_t stream) {
    if (in_f32)
        return out_f32 ? launch_state_xy_t<D, true, true>(B, T, H, NC, scale, ws, S0, ST, o, cr, stream)
                       : launch_state_xy_t<D, true, false>(B, T, H, NC, scale, ws, S0, ST, o, cr, stream);
    return out_f32 ? launch_state_xy_t<D, false, true>(B, T, H, NC, scale, ws, S0, ST, o, cr, stream)
                   : launch_state_xy_t<D, false, false>(B, T, H, NC, scale, ws, S0, ST, o, cr, stream);
}

hipError_t launch_state_fwd_xy(int D, bool in_f32, bool out_f32, int64_t B, int64_t T, int H, int64_t NC,
                               float scale, const ChunkWs& ws, const float* S0, float* ST, void* o, ChunkRange cr,
                               hipStream_t stream) {
    if (D == 64) return launch_state_xy_d<64>(in_f32, out_f32, B, T, H, NC, scale, ws, S0, ST, o, cr, stream);
    return launch_state_xy_d<128>(in_f32, out_f32, B, T, H, NC, scale, ws, S0, ST, o, cr, stream);
}

hipError_t launch_state_fwd(int D, bool in_f32, bool out_f32, int64_t B, int64_t T, int H,
                            int64_t NC, float scale, const ChunkWs& ws, const float* S0,
                            float* ST, void* o, bool save_for_backward, bool wide, ChunkRange cr, hipStream_t stream) {
    if (D == 64) {
        if (in_f32) {
            if (out_f32) return launch_state_t<64, true, true>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, wide, cr, stream);
            return launch_state_t<64, true, false>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, wide, cr, stream);
        }
        if (out_f32) return launch_state_t<64, false, true>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, wide, cr, stream);
        return launch_state_t<64, false, false>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, wide, cr, stream);
    }
    if (in_f32) {
        if (out_f32) return launch_state_t<128, true, true>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, wide, cr, stream);
        return launch_state_t<128, true, false>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, wide, cr, stream);
    }
    if (out_f32) return launch_state_t<128, false, true>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, wide, cr, stream);
    return launch_state_t<128, false, false>(B, T, H, NC, scale, ws, S0, ST, o, save_for_backward, wide, cr, stream);
}

}  // namespace gdr
