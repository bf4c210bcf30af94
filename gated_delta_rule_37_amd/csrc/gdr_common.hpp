// gdr_common.hpp -- shared device helpers for the gfx950 kernels of libgdr.
//
// Matrix-core (MFMA) fragments.  Every product in the chunked path is tiled
// into 16x16 output tiles contracted over K in steps of 32:
//   A fragment (16 x 32, row-major M x K): lane l holds row (l % 16) and the
//     eight consecutive k = 8*(l/16) .. 8*(l/16)+7.
//   B fragment (32 x 16, K x N): lane l holds column (l % 16) and the same
//     eight consecutive k.
//   C/D tile (16 x 16, fp32): lane l holds column (l % 16) and rows
//     4*(l/16) .. 4*(l/16)+3.
// For fp16 operands one v_mfma_f32_16x16x32_f16 consumes a fragment pair.  For
// fp32 operands the same fragments feed eight v_mfma_f32_16x16x4_f32: the i-th
// instruction takes element i of every lane, so lane group g contributes
// k = 8g + i.  A contraction only needs A and B to agree on the k order, so both
// precisions share one fragment layout and one set of address computations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float8v __attribute__((ext_vector_type(8)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // raw bfloat16 bits

enum Gate { GATE_NONE = 0, GATE_SCALAR = 1, GATE_CHANNEL = 2 };

constexpr int WAVE = 64;
constexpr int CHUNK = 64;

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN kept quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<bf16_t>((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

// Element type of the inputs: bf16 (raw bits) or fp32.
template <bool F32> struct InType { using T = bf16_t; };
template <> struct InType<true> { using T = float; };

__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }
// The empty asm pins x as an fp32 value: without it the compiler may fuse a
// product feeding the conversion into one mixed-precision FMA (one rounding
// instead of two), and whether it does depends on the surrounding code, so two
// kernels computing the same value could round it differently.  The asm is not
// volatile: it has no side effects, so memory accesses may still be scheduled
// across it (a volatile one kept every load after a conversion from being
// issued before it).
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) {
    asm("" : "+v"(x));
    return static_cast<_Float16>(x);
}

// ---------------------------------------------------------------------------
// MFMA fragments
// ---------------------------------------------------------------------------

template <typename OpT> struct Frag;

template <> struct Frag<_Float16> {
    half8 v;
    __device__ __forceinline__ void zero() {
        for (int i = 0; i < 8; ++i) v[i] = static_cast<_Float16>(0.f);
    }
    __device__ __forceinline__ void load(const _Float16* p) { v = *reinterpret_cast<const half8*>(p); }
};

template <> struct Frag<float> {
    float8v v;
    __device__ __forceinline__ void zero() {
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    __device__ __forceinline__ void load(const float* p) {
        const float4v a = reinterpret_cast<const float4v*>(p)[0];
        const float4v b = reinterpret_cast<const float4v*>(p)[1];
        v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
        v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    }
};

// acc += A(16x32) * B(32x16)
__device__ __forceinline__ void mma(const Frag<_Float16>& a, const Frag<_Float16>& b, float4v& acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(const Frag<float>& a, const Frag<float>& b, float4v& acc) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
}

// Fragment-order storage.  A matrix that a later kernel reads as MFMA A or B
// operands is written so that every 64-lane fragment is one contiguous block
// (lane l's eight k-consecutive elements at [frag][l][0..7]); a load
// instruction then reads 64 x 16 contiguous bytes instead of 16-byte pieces of
// 16 different rows.  frag_off gives the element offset of (r, k) in an
// M x K operand; cfrag_off the offset of (r, n) in an M x N matrix stored in
// accumulator order (lane l holding rows 4(l/16)..+3 of column l%16).
template <int K>
__host__ __device__ __forceinline__ int frag_off(int r, int k) {
    const int rt = r >> 4, l16 = r & 15, kq = k >> 5, g = (k >> 3) & 3, e = k & 7;
    return ((rt * (K / 32) + kq) * 64 + g * 16 + l16) * 8 + e;
}
template <int N>
__host__ __device__ __forceinline__ int cfrag_off(int r, int n) {
    const int rt = r >> 4, ct = n >> 4, lane = ((r & 15) >> 2) * 16 + (n & 15), e = r & 3;
    return ((rt * (N / 16) + ct) * 64 + lane) * 4 + e;
}

__device__ __forceinline__ float4v zero4() {
    float4v z;
    z[0] = 0.f; z[1] = 0.f; z[2] = 0.f; z[3] = 0.f;
    return z;
}

// Stores N consecutive values (16-byte aligned destination) in operand precision.
template <typename OpT, int N>
__device__ __forceinline__ void store_run(OpT* dst, const float* src) {
    // N consecutive values, 16-byte aligned destination
    if constexpr (sizeof(OpT) == 2) {
#pragma unroll
        for (int i = 0; i < N; i += 8) {
            half8 h;
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = from_f32<_Float16>(src[i + e]);
            *reinterpret_cast<half8*>(dst + i) = h;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            float4v f;
#pragma unroll
            for (int e = 0; e < 4; ++e) f[e] = src[i + e];
            *reinterpret_cast<float4v*>(dst + i) = f;
        }
    }
}

// Stores the four values of an accumulator quad in operand precision.
template <typename OpT>
__device__ __forceinline__ void store4(OpT* dst, const float4v& v) {
    if constexpr (sizeof(OpT) == 2) {
        half4 h;
        h[0] = from_f32<_Float16>(v[0]); h[1] = from_f32<_Float16>(v[1]);
        h[2] = from_f32<_Float16>(v[2]); h[3] = from_f32<_Float16>(v[3]);
        *reinterpret_cast<half4*>(dst) = h;
    } else {
        *reinterpret_cast<float4v*>(dst) = v;
    }
}


// Column piece of an LDS array: out[e] = t[off(r0 + e, c0 + lane % 16)],
// e = 0..7, where off(r, c) is the element offset of row r, column c, the 16
// lanes of a group share r0 and c0 (so a group reads 16 consecutive columns)
// and all 16 take part.  16-bit elements (moved as raw bits): two gfx950
// transposed reads (ds_read_b64_tr_b16), which hand lane 4a+i of a 16-lane
// group element i of the 8-byte pieces that lanes a, a+4, a+8 and a+12 of the
// group address; so lane c addresses row r0 + c/4 (+4 in the second read),
// columns c0 + 4(c%4) .. +3, which must be four consecutive, 8-byte aligned
// elements (c0 a multiple of 16; true of a row-major array with a row stride
// that is a multiple of 4, and of the fragment order).  fp32: eight plain reads.
// t may point to LDS generically or in the LDS address space.
template <typename Ptr, typename T, typename Off>
__device__ __forceinline__ void lds_column8_at(Ptr t, int r0, int c0, int lane, Off off, T (&out)[8]) {
    if constexpr (sizeof(T) == 2) {
        typedef short short4v __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) short4v lds_short4;
        const int c = lane & 15, r = r0 + (c >> 2), cc = c0 + 4 * (c & 3);
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(t + off(r, cc)));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(t + off(r + 4, cc)));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            out[e] = __builtin_bit_cast(T, static_cast<short>(lo[e]));
            out[4 + e] = __builtin_bit_cast(T, static_cast<short>(hi[e]));
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = t[off(r0 + e, c0 + (lane & 15))];
    }
}

// The same for a row-major array with row stride LD elements.
template <int LD, typename OpT>
__device__ __forceinline__ void lds_column8(const OpT* t, int r0, int c0, int lane, OpT (&out)[8]) {
    static_assert(LD % 4 == 0, "8-byte aligned pieces");
    lds_column8_at(t, r0, c0, lane, [](int r, int c) { return r * LD + c; }, out);
}

// ---------------------------------------------------------------------------
// direct global -> LDS copies (global_load_lds) and explicit vmcnt waits
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) char lds_char;  // byte pointer into LDS

// Each lane copies 16 bytes from src_lane + OFF to lds_base + OFF + 16 * lane
// (the instruction offset applies to both addresses).  lds_base must be the
// same for the whole wave.  The copy is counted by vmcnt and the data is in
// LDS once the wave's vmcnt has dropped past it.
template <int OFF = 0>
__device__ __forceinline__ void copy16_to_lds(const void* src_lane, lds_char* lds_base) {
    __builtin_amdgcn_global_load_lds(src_lane, (lds_ptr_t)lds_base, 16, OFF, 0);
}
// Each lane copies 4 bytes (used to pull lines into the L2).
__device__ __forceinline__ void copy4_to_lds(const void* src_lane, lds_char* lds_base) {
    __builtin_amdgcn_global_load_lds(src_lane, (lds_ptr_t)lds_base, 4, 0, 0);
}
// A contiguous block of NKB KiB, one wave: four 1 KiB copies per address.
template <int NKB>
__device__ __forceinline__ void copy_block_to_lds(const char* src, lds_char* dst, int lane) {
#pragma unroll
    for (int i = 0; i < NKB; i += 4) {
        const char* s = src + i * 1024 + lane * 16;
        lds_char* d = dst + i * 1024;
        copy16_to_lds<0>(s, d);
        if (i + 1 < NKB) copy16_to_lds<1024>(s, d);
        if (i + 2 < NKB) copy16_to_lds<2048>(s, d);
        if (i + 3 < NKB) copy16_to_lds<3072>(s, d);
    }
}

// s_waitcnt vmcnt(N), leaving the other counters alone (gfx9 encoding: vmcnt
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | 0x0F70 | (N & 15));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / WAVE; }

// Eight consecutive values (16-byte aligned) converted to / from fp32.
template <typename T>
__device__ __forceinline__ void load8f(const T* p, float (&x)[8]) {
    if constexpr (sizeof(T) == 2) {
        const uint4 r = *reinterpret_cast<const uint4*>(p);
        const T* v = reinterpret_cast<const T*>(&r);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = to_f32(v[e]);
    } else {
        const float4v a = reinterpret_cast<const float4v*>(p)[0];
        const float4v b = reinterpret_cast<const float4v*>(p)[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = a[e];
            x[4 + e] = b[e];
        }
    }
}

template <typename T>
__device__ __forceinline__ void store8f(T* p, const float (&x)[8]) {
    if constexpr (sizeof(T) == 2) {
        uint4 r;
        T* v = reinterpret_cast<T*>(&r);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = from_f32<T>(x[e]);
        *reinterpret_cast<uint4*>(p) = r;
    } else {
        float4v a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = x[e];
            b[e] = x[4 + e];
        }
        reinterpret_cast<float4v*>(p)[0] = a;
        reinterpret_cast<float4v*>(p)[1] = b;
    }
}

// lam[c..c+7], or ones when lam is NULL (the unit scale)
__device__ __forceinline__ void load_lam8(const float* lam, int64_t c, float (&x)[8]) {
    if (lam) {
        const float4v a = *reinterpret_cast<const float4v*>(lam + c);
        const float4v b = *reinterpret_cast<const float4v*>(lam + c + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = a[e];
            x[4 + e] = b[e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 1.f;
    }
}

// Fast base-2 exponent and logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Prefix sums over a chunk of one value per row (row = lane of one 64-lane
// wave), associated the way the per-channel path sums a column: a running sum
// inside each 16-row block, then the totals of the earlier blocks added in
// order.  The difference of two prefixes then carries the rounding of the terms
// between them only (not that of the whole prefix), and rows that add 0 repeat
// the previous prefix exactly, so a chunk's last prefix equals that of its last
// valid row.  All 64 lanes must call it.
__device__ __forceinline__ float chunk_prefix_sum(float x) {
    const int lane = threadIdx.x & 63, li = lane & 15, blk = lane >> 4;
    float s = x;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
        const float prev = __shfl_up(s, 1);
        s = (li == i) ? prev + x : s;
    }
    const float t0 = __shfl(s, 15), t1 = __shfl(s, 31), t2 = __shfl(s, 47);
    float carry = 0.f;
    carry += blk > 0 ? t0 : 0.f;
    carry += blk > 1 ? t1 : 0.f;
    carry += blk > 2 ? t2 : 0.f;
    return s + carry;
}

// ---------------------------------------------------------------------------
// Prologue: L2-normalised q and k, activated gates (KDA blog, sections 2.1 and
// 7.1: an L2 norm after the q/k projections; sigmoid gates, with the forget
// gate's logit biased to -3 so that it forgets ~5 % per token at the start).
//   PRO 1: beta = sigmoid(b), alpha = sigmoid(a)
//   PRO 2: beta = sigmoid(b), alpha = exp(-softplus(a)) = sigmoid(-a)
// A row is divided by max(|row|_2, NORM_EPS).
// ---------------------------------------------------------------------------
constexpr float NORM_EPS = 1e-6f;

// sigmoid with the hardware exp2; 1 - sigmoid(x) is sigmoid(-x), never formed
// by subtraction
__device__ __forceinline__ float sigmoid_fast(float x) {
    return __builtin_amdgcn_rcpf(1.f + exp2_fast(-x * 1.4426950408889634f));
}

// s = +1 (PRO 1) or -1 (PRO 2): alpha = sigmoid(s a)
__device__ __forceinline__ float pro_sign(int pro) { return pro == 1 ? 1.f : -1.f; }

// log2(alpha) from the logit without forming alpha:
//   log2 sigmoid(s a) = -log2(1 + 2^(-s a log2 e))
//                     = -(max(y, 0) + log2(1 + 2^-|y|)),  y = -s a log2 e.
// Where 2^-|y| is below fp32's half ulp of 1 the second term is lost: an
// absolute error below 2^-24 in log2(alpha), i.e. alpha within an ulp of 1.
__device__ __forceinline__ float log2_alpha_logit(float a, int pro) {
    const float y = -pro_sign(pro) * a * 1.4426950408889634f;
    return -(fmaxf(y, 0.f) + log2_fast(1.f + exp2_fast(-fabsf(y))));
}

// d alpha-logit from the gradient with respect to ln(alpha):
// d ln(sigmoid(s a)) / da = s (1 - sigmoid(s a)) = s sigmoid(-s a)
__device__ __forceinline__ float dlogit_from_dlog(float dlog, float a, int pro) {
    const float s = pro_sign(pro);
    return dlog * s * sigmoid_fast(-s * a);
}

// Reciprocal norm of a row, with the clamped case flagged by the sign (the
// gradient then has no projection term).
__device__ __forceinline__ float recip_norm(float sumsq) {
    return sumsq > NORM_EPS * NORM_EPS ? __builtin_amdgcn_rsqf(sumsq) : -1.f / NORM_EPS;
}

// Sums x[j] (32 values per thread) over the D threads of this thread's part
// (threads part*D .. part*D + D - 1, D / 64 whole waves) for every j; every
// thread of the part receives the 32 totals.  A butterfly that halves the
// values each step (reduce-scatter: 16 + 8 + 4 + 2 + 1 + 1 exchanges instead of
// 32 * 6) leaves lane l with the wave's sum of value (l >> 1) & 31; the sums
// go through LDS.  The order of additions is fixed.  red: LDS scratch of
// (threads / 64) * 32 floats.  Called by every thread of the workgroup.
// One butterfly step: lanes with bit M keep the upper N/2 values, their
// partners the lower ones; each receives the other half from its partner.
template <int N, int M>
__device__ __forceinline__ void butterfly_step(float (&x)[32], int lane) {
    const bool up = (lane & M) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        const float send = up ? x[i] : x[i + N / 2];
        const float keep = up ? x[i + N / 2] : x[i];
        x[i] = keep + __shfl_xor(send, M);
    }
}

template <int D>
__device__ __forceinline__ void part_row_sums32(float (&x)[32], float* red) {
    const int lane = threadIdx.x & (WAVE - 1), wid = threadIdx.x / WAVE;
    butterfly_step<32, 32>(x, lane);
    butterfly_step<16, 16>(x, lane);
    butterfly_step<8, 8>(x, lane);
    butterfly_step<4, 4>(x, lane);
    butterfly_step<2, 2>(x, lane);
    x[0] += __shfl_xor(x[0], 1);
    if ((lane & 1) == 0) red[wid * 32 + ((lane >> 1) & 31)] = x[0];
    __syncthreads();
    if constexpr (D == WAVE) {
#pragma unroll
        for (int j = 0; j < 32; ++j) x[j] = red[wid * 32 + j];
    } else {
        static_assert(D == 2 * WAVE, "two waves per part");
        const int w0 = wid & ~1;
#pragma unroll
        for (int j = 0; j < 32; ++j) x[j] = red[w0 * 32 + j] + red[(w0 + 1) * 32 + j];
    }
    __syncthreads();
}

}  // namespace gdr
