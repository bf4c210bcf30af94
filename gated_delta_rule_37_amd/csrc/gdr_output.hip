// gdr_output.hip -- chunk outputs from the saved chunk-start states.
//
// With S the state at the start of chunk c (as the chain pass saved it) and U
// the chunk's beta-scaled write errors, every output row of the chunk is
//   O = scale (Qt S + A U)
// (read-out after each token's write, KDA blog section 2.1, in the chunked form
// of section 6.1).  None of this is sequential, so it runs over all chunk-heads
// at once, one workgroup each.
//
// The saved S and U are in the fragment order the gradient kernels read (rows
// d resp. position, k = value column).  Here the contraction runs over d resp.
// position: both are laid out row-major in LDS (one 16-byte store per saved
// piece) and read back as B fragments with the transposed LDS read, so no
// element is moved on its own; Qt and A are copied to LDS as they are.  Wave w
// owns the value columns 32w..32w+31 of all 64 rows.  The products accumulate
// in the same order as a fused state pass would (Qt S over d, then A U), in
// fp32.
//
// With the error-routing epilogue (CLER), every thread also adds lam * u / beta
// to the hidden-stream piece of the U piece it has just read (the write errors,
// see gdr_cler.hpp), so U is read once for both.
//
// With the output-gate epilogue (GATE, KDA blog section 4.1), the rows
// assembled in LDS are not written as o: each is normalised over its dv
// channels, scaled by w and by sigmoid(g), and written as y.  The lanes own the
// same eight channels of a row, and the norm reduces in the same order, as in
// gate_fwd_kernel, so y equals that kernel run on o, bit for bit, without o
// being written and read back.  g is loaded before the products, so its reads
// overlap them.
#include "gdr_cler.hpp"
#include "gdr_common.hpp"
#include "gdr_gate_rows.hpp"
#include "gdr_launch.hpp"

namespace gdr {

template <int D>
struct OutLayout {
    static constexpr int LDR = D + 8;       // row stride of S [D][D] and U [64][D] (fp16)
    static constexpr int ST = 0;
    static constexpr int UT = ST + D * LDR * 2;
    static constexpr int QT = UT + CHUNK * LDR * 2;  // Qt, fragment order copy
    static constexpr int A = QT + CHUNK * D * 2;     // A, fragment order copy
    static constexpr int BYTES = A + CHUNK * CHUNK * 2;
};

// B fragment (k = row, n = column) of a row-major fp16 tile in LDS: lane l gets
// rows k0 + 8(l/16) .. +7 of column n0 + l%16.
template <int LD>
__device__ __forceinline__ Frag<_Float16> frag_tr(const _Float16* t, int k0, int n0, int lane) {
    _Float16 x[8];
    lds_column8<LD>(t, k0 + 8 * (lane >> 4), n0, lane, x);
    Frag<_Float16> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = x[e];
    return f;
}

template <int D, bool OUT_F32, bool CLER, bool GATE>
__global__ __launch_bounds__(256) void output_kernel(int64_t T, int H, int64_t NC, float scale, ChunkWs ws,
                                                     void* __restrict__ o_, const float* __restrict__ beta,
                                                     const float* __restrict__ lam, bf16_t* __restrict__ hs,
                                                     const bf16_t* __restrict__ gg, const float* __restrict__ gw,
                                                     ChunkRange cr) {
    using L = OutLayout<D>;
    using OutT = typename InType<OUT_F32>::T;
    constexpr int LDR = L::LDR;
    constexpr int CPW = D / 4 / 16;  // column tiles per wave

    __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];
    _Float16* sS = reinterpret_cast<_Float16*>(smem + L::ST);
    _Float16* sU = reinterpret_cast<_Float16*>(smem + L::UT);

    int64_t bh, c;
    range_block(cr, bh, c);
    const int64_t ch = bh * NC + c;
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh % H);
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t nvalid64 = T - c * CHUNK;
    const int nvalid = nvalid64 < CHUNK ? static_cast<int>(nvalid64) : CHUNK;

    // Qt and A: straight copies (fragment order), 1 KiB per copy
    {
        const char* Qg = static_cast<const char*>(ws.Qt) + ch * CHUNK * D * 2;
        const char* Ag = static_cast<const char*>(ws.A) + ch * CHUNK * CHUNK * 2;
        constexpr int NQ = CHUNK * D * 2 / 1024, NA = CHUNK * CHUNK * 2 / 1024;
        for (int i = wid; i < NQ + NA; i += 4) {
            lds_char* sm = (lds_char*)&smem[0];
            if (i < NQ) copy16_to_lds(Qg + i * 1024 + lane * 16, sm + L::QT + i * 1024);
            else copy16_to_lds(Ag + (i - NQ) * 1024 + lane * 16, sm + L::A + (i - NQ) * 1024);
        }
    }
    // S and U row-major: piece p of a fragment-ordered [M][D] array is lane
    // (p % 64) of fragment p / 64 = (row tile, 32-column step), eight
    // consecutive columns of one row
    {
        const _Float16* Sg = reinterpret_cast<const _Float16*>(ws.Ssnap) + ch * D * D;
        const _Float16* Ug = reinterpret_cast<const _Float16*>(ws.Usave) + ch * CHUNK * D;
#pragma unroll
        for (int i = 0; i < D * D / 8 / 256; ++i) {
            const int p = i * 256 + tid, f = p >> 6, l = p & 63;
            const int d = 16 * (f / (D / 32)) + (l & 15), j = 32 * (f % (D / 32)) + 8 * (l >> 4);
            *reinterpret_cast<half8*>(sS + d * LDR + j) = *reinterpret_cast<const half8*>(Sg + p * 8);
        }
#pragma unroll
        for (int i = 0; i < CHUNK * D / 8 / 256; ++i) {
            const int p = i * 256 + tid, f = p >> 6, l = p & 63;
            const int pos = 16 * (f / (D / 32)) + (l & 15), j = 32 * (f % (D / 32)) + 8 * (l >> 4);
            const half8 v = *reinterpret_cast<const half8*>(Ug + p * 8);
            *reinterpret_cast<half8*>(sU + pos * LDR + j) = v;
            if constexpr (CLER) {
                if (pos < nvalid) {
                    const int64_t t = c * CHUNK + pos;
                    float u[8], lm[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) u[e] = static_cast<float>(v[e]);
                    load_lam8(lam, static_cast<int64_t>(h) * D + j, lm);
                    cler_add8(hs + ((b * T + t) * H + h) * D + j, u, lm, beta[(b * T + t) * H + h]);
                }
            }
        }
    }
    const int64_t tstride = static_cast<int64_t>(H) * D;
    const int64_t obase = ((b * T + c * CHUNK) * H + h) * D;
    // output gate: TPR lanes per row, eight channels each; rows past the end
    // are neither read nor written
    constexpr int TPR = D / 8, RPI = 256 / TPR, GR = GATE ? CHUNK / RPI : 1;
    const int grs = tid / TPR, gc0 = (tid % TPR) * 8;
    uint4 graw[GR];
    if constexpr (GATE) {
#pragma unroll
        for (int k = 0; k < GR; ++k) {
            const int r = k * RPI + grs;
            graw[k] = r < nvalid ? *reinterpret_cast<const uint4*>(gg + obase + r * tstride + gc0) : make_uint4(0, 0, 0, 0);
        }
    }
    wait_vmcnt<0>();
    __syncthreads();
    OutT* o = reinterpret_cast<OutT*>(o_);
    float res[4][CPW][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        Frag<_Float16> fq[D / 32], fa[2];
#pragma unroll
        for (int kq = 0; kq < D / 32; ++kq)
            fq[kq].v = *reinterpret_cast<const half8*>(smem + L::QT + ((rt * (D / 32) + kq) * 64 + lane) * 16);
        fa[0].v = *reinterpret_cast<const half8*>(smem + L::A + ((rt * 2 + 0) * 64 + lane) * 16);
        fa[1].v = *reinterpret_cast<const half8*>(smem + L::A + ((rt * 2 + 1) * 64 + lane) * 16);
#pragma unroll
        for (int ci = 0; ci < CPW; ++ci) {
            const int ct = wid * CPW + ci;
            float4v acc = zero4();
#pragma unroll
            for (int kq = 0; kq < D / 32; ++kq) {
                mma(fq[kq], frag_tr<LDR>(sS, 32 * kq, 16 * ct, lane), acc);
            }
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                mma(fa[kq], frag_tr<LDR>(sU, 32 * kq, 16 * ct, lane), acc);  // the upper blocks of A are zero
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) res[rt][ci][e] = scale * acc[e];
        }
    }
    // assemble the output rows in LDS (over S, no longer read) and write them
    // with 16-byte stores; rows past the end are not written
    __syncthreads();
    static_assert(CHUNK * D * sizeof(OutT) <= L::QT, "output rows must fit over S and U");
    OutT* so = reinterpret_cast<OutT*>(smem + L::ST);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ci = 0; ci < CPW; ++ci)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                so[(16 * rt + 4 * g4 + e) * D + 16 * (wid * CPW + ci) + l16] = from_f32<OutT>(res[rt][ci][e]);
    __syncthreads();
    if constexpr (GATE) {
        float wv[8];
        load_lam8(gw, static_cast<int64_t>(h) * D + gc0, wv);
#pragma unroll
        for (int k = 0; k < GR; ++k) {
            const int r = k * RPI + grs;
            float ov[8], gv[8];
            load8f(so + r * D + gc0, ov);
            const bf16_t* gb = reinterpret_cast<const bf16_t*>(&graw[k]);
#pragma unroll
            for (int i = 0; i < 8; ++i) gv[i] = to_f32(gb[i]);
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(ov[i], ov[i], ss);
            ss = row_sum<TPR>(ss);
            const float rstd = __builtin_amdgcn_rsqf(ss * (1.f / D) + GATE_EPS);
            float yv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) yv[i] = sigmoid_fast(gv[i]) * wv[i] * (ov[i] * rstd);
            if (r < nvalid) store8f(o + obase + r * tstride + gc0, yv);
        }
        return;
    }
    constexpr int EPP = 16 / sizeof(OutT);      // elements per 16-byte piece
    constexpr int PPR = D / EPP;                // pieces per row
    constexpr int NPC = CHUNK * PPR / 256;      // pieces per thread
#pragma unroll
    for (int k2 = 0; k2 < NPC; ++k2) {
        const int p = k2 * 256 + tid, r = p / PPR, c0 = (p % PPR) * EPP;
        if (r < nvalid)
            *reinterpret_cast<uint4*>(o + obase + r * tstride + c0) = *reinterpret_cast<const uint4*>(so + r * D + c0);
    }
}

template <int D, bool OUT_F32, bool CLER>
static void launch_output_g(int64_t nch, int64_t T, int H, int64_t NC, float scale, const ChunkWs& ws, void* o,
                            const float* beta, const float* lam, bf16_t* hs, const OutGate& og, ChunkRange cr,
                            hipStream_t stream) {
    const bf16_t* gg = static_cast<const bf16_t*>(og.g);
    if (gg)
        hipLaunchKernelGGL((output_kernel<D, OUT_F32, CLER, true>), dim3((unsigned)nch), dim3(256), 0, stream, T, H,
                           NC, scale, ws, o, beta, lam, hs, gg, og.w, cr);
    else
        hipLaunchKernelGGL((output_kernel<D, OUT_F32, CLER, false>), dim3((unsigned)nch), dim3(256), 0, stream, T,
                           H, NC, scale, ws, o, beta, lam, hs, gg, og.w, cr);
}

template <int D, bool OUT_F32>
static void launch_output_t(int64_t nch, int64_t T, int H, int64_t NC, float scale, const ChunkWs& ws, void* o,
                            const float* beta, const float* lam, void* h, const OutGate& og, ChunkRange cr,
                            hipStream_t stream) {
    bf16_t* hs = static_cast<bf16_t*>(h);
    if (h) launch_output_g<D, OUT_F32, true>(nch, T, H, NC, scale, ws, o, beta, lam, hs, og, cr, stream);
    else launch_output_g<D, OUT_F32, false>(nch, T, H, NC, scale, ws, o, beta, lam, hs, og, cr, stream);
}

static hipError_t launch_output_any(int D, bool out_f32, int64_t B, int64_t T, int H, int64_t NC, float scale,
                                    const ChunkWs& ws, void* o, const float* beta, const float* lam, void* h_cler,
                                    const OutGate& og, ChunkRange cr, hipStream_t stream) {
    const int64_t nch = B * H * cr.n;
    if (nch == 0) return hipSuccess;
    if (D == 64) {
        if (out_f32) launch_output_t<64, true>(nch, T, H, NC, scale, ws, o, beta, lam, h_cler, og, cr, stream);
        else launch_output_t<64, false>(nch, T, H, NC, scale, ws, o, beta, lam, h_cler, og, cr, stream);
    } else {
        if (out_f32) launch_output_t<128, true>(nch, T, H, NC, scale, ws, o, beta, lam, h_cler, og, cr, stream);
        else launch_output_t<128, false>(nch, T, H, NC, scale, ws, o, beta, lam, h_cler, og, cr, stream);
    }
    return hipGetLastError();
}

hipError_t launch_output(int D, bool out_f32, int64_t B, int64_t T, int H, int64_t NC, float scale,
                         const ChunkWs& ws, void* o, const float* beta, const float* lam, void* h_cler,
                         ChunkRange cr, hipStream_t stream) {
    return launch_output_any(D, out_f32, B, T, H, NC, scale, ws, o, beta, lam, h_cler, OutGate{nullptr, nullptr},
                             cr, stream);
}

hipError_t launch_output_gated(int D, bool out_f32, int64_t B, int64_t T, int H, int64_t NC, float scale,
                               const ChunkWs& ws, void* o, const float* beta, const float* lam, void* h_cler,
                               const OutGate& og, ChunkRange cr, hipStream_t stream) {
    return launch_output_any(D, out_f32, B, T, H, NC, scale, ws, o, beta, lam, h_cler, og, cr, stream);
}

}  // namespace gdr
