// gdr_abi.cpp -- the C ABI of libgdr (declared in include/gdr.h).
//
// Host code only: argument validation (pure functions of sizes and pointer
// values, so it runs and is tested without a GPU), workspace sizing and carving,
// and kernel launches on the caller's stream.  No function here allocates
// device memory, throws or aborts; none synchronises except in the debug mode
// (GDR_VALIDATE=1), which checks the inputs on the device first.
#include "../../include/gdr.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "gdr_gate.hpp"
#include "gdr_launch.hpp"

namespace {

thread_local char g_err[512] = "";

gdr_status fail(gdr_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

constexpr int kChunk = 64;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [p, p+n) and [q, q+m) share a byte
bool overlap(const void* p, size_t n, const void* q, size_t m) {
    if (!p || !q || n == 0 || m == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + m && b < a + n;
}

size_t dtype_bytes(int32_t dt) { return dt == GDR_FP32 ? 4 : 2; }

// ---------------------------------------------------------------------------
// Overlap of the sequential state passes with per-chunk work.  A state pass
// runs one workgroup per (batch, head, 16-column slice); when that leaves CUs
// idle, the pass is cut into chunk ranges (its state handed from one launch to
// the next through the workspace) and the per-chunk kernels of a finished range
// run on a second stream while the pass continues.  The second stream and the
// events that order it against the caller's stream are created once per device
// (default priority) and reused; enqueueing is serialised by a mutex so that
// concurrent callers never interleave their uses of the shared events.
// ---------------------------------------------------------------------------
constexpr int kAuxEvents = 16;
constexpr int kMaxDevices = 64;

struct Aux {
    hipStream_t s = nullptr, s2 = nullptr;  // s2: the forward's outputs while s runs intra-chunk ranges
    hipEvent_t ev[kAuxEvents] = {};
    int cus = 0;
    bool ok = false, tried = false;
};
std::mutex g_aux_mu;
Aux g_aux[kMaxDevices];

// The current device's second stream, or nullptr if it cannot be had (then
// everything runs on the caller's stream).  Call with g_aux_mu held.
Aux* aux_stream() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    Aux& a = g_aux[dev];
    if (!a.tried) {
        a.tried = true;
        hipDeviceProp_t prop;
        bool ok = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                  hipStreamCreateWithFlags(&a.s, hipStreamNonBlocking) == hipSuccess &&
                  hipStreamCreateWithFlags(&a.s2, hipStreamNonBlocking) == hipSuccess;
        for (int i = 0; ok && i < kAuxEvents; ++i)
            ok = hipEventCreateWithFlags(&a.ev[i], hipEventDisableTiming) == hipSuccess;
        a.cus = ok ? prop.multiProcessorCount : 0;
        a.ok = ok;
    }
    return a.ok ? &a : nullptr;
}

// Ranges to cut a state pass of `blocks` workgroups over NC chunks into: one
// while the pass fills the chip, else up to kMaxParts of at least 16 chunks.
// (At the 32K-token KDA shape the training step took 3.37, 3.34, 3.41 and
// 3.55 ms with at most 2, 4, 8 and 16 ranges: more ranges add relaunch and
// pipeline-fill costs and shrink the grids of the overlapped kernels.)
constexpr int kMaxParts = 4;
static_assert(2 * kMaxParts < kAuxEvents, "events of a cut forward");
// How far ahead the gradient kernel prefetches (launch_grads): five sixths of
// the CUs it gets, a multiple of the 8 XCDs.  A workgroup issues the prefetch
// about halfway through its run, so the workgroup that many places later
// starts soon after on the same XCD (at the 32K-token KDA shape, 192 CUs beside
// the reverse pass: 2.42 against 2.47 ms per training step, and 2.43, 2.45,
// 2.44 and 2.46 ms at 128, 192, 224 and 256 places).
int grads_ahead(const Aux* a, int64_t busy) {
    const int64_t avail = a ? a->cus - busy : 0;
    if (avail < 16) return 0;
    return static_cast<int>(avail * 5 / 6) & ~7;
}

int state_parts(const Aux* a, int64_t blocks, int64_t NC) {
    if (!a || blocks >= a->cus) return 1;
    const int64_t p = NC / 16;
    return int(p < 1 ? 1 : (p > kMaxParts ? kMaxParts : p));
}

// Bounds of range p of a pass cut into `parts`, in the order the pass runs.
// Range sizes grow geometrically (weights 1 : r : r^2 : ..., r = ra / rb) away from the
// range whose per-chunk work cannot overlap anything: the first range of the
// reverse pass (its gradient kernels wait for it, and each later range should
// be ready about when the gradient kernels of the one before finish, which run
// longer per chunk than the chain on the CUs it leaves them) and the last range
// of the forward (its output kernel runs after the chain).  A range keeps at
// least 16 chunks where the sizes allow.  (At the 32K-token KDA shape, ratios
// 2, 3/2 and 1.3 between neighbours gave 2.90, 2.89 and 2.92 ms per training
// step, equal ranges 3.04 ms.  With the forward's intra-chunk ranges overlapping
// the chain, its largest-first order still measured best: inference forward
// 1.01 ms against 1.07 smallest first and 1.06 with equal ranges.  Measured
// again at 2.48 ms per step: 3, 5 or 6 ranges and ratios 4/3 and 5/3 all
// slower for the training step, by 0.3-2.7 %; the inference forward alone is
// 2.5 % faster with r = 4/3, which it uses: 0.869 against 0.892 ms.)
void cut_range(int64_t NC, int parts, int p, bool reverse, int64_t* lo, int64_t* hi, int ra, int rb) {
    if (parts < 2) {
        *lo = 0;
        *hi = NC;
        return;
    }
    // sizes in processing order for the reverse pass: w_i = ra^i rb^(parts-1-i)
    int64_t size[kMaxParts], w[kMaxParts];
    int64_t wsum = 0;
    for (int i = 0; i < parts; ++i) {
        w[i] = 1;
        for (int j = 0; j < parts - 1; ++j) w[i] *= j < i ? ra : rb;
        wsum += w[i];
    }
    int64_t used = 0;
    for (int i = 0; i < parts; ++i) {
        int64_t n = NC * w[i] / wsum;
        if (n < 16) n = 16;
        size[i] = n;
        used += n;
    }
    size[parts - 1] += NC - used;  // the largest range absorbs the remainder
    if (size[parts - 1] < 1) {
        // the minimums left nothing for it: equal ranges instead
        for (int i = 0; i < parts; ++i) size[i] = NC / parts + (i < NC % parts ? 1 : 0);
    }
    // range i of the reverse order covers the chunks from the top down; the
    // forward uses the same sizes from chunk 0 up, largest first
    const int i = reverse ? p : parts - 1 - p;
    int64_t top = NC;
    for (int j = 0; j < i; ++j) top -= size[j];
    *hi = top;
    *lo = top - size[i];
}

// Checks a descriptor; fills derived sizes.
gdr_status check_desc(const gdr_desc* d, int64_t* NC) {
    if (!d) return fail(GDR_ERR_INVALID_ARG, "desc is NULL");
    if (d->B < 0 || d->T < 0 || d->H < 0)
        return fail(GDR_ERR_INVALID_ARG, "B, T, H must be >= 0 (got %lld, %lld, %lld)",
                    (long long)d->B, (long long)d->T, (long long)d->H);
    if (d->gate < GDR_GATE_NONE || d->gate > GDR_GATE_CHANNEL)
        return fail(GDR_ERR_INVALID_ARG, "unknown gate kind %d", d->gate);
    if ((d->in_dtype != GDR_BF16 && d->in_dtype != GDR_FP32) ||
        (d->out_dtype != GDR_BF16 && d->out_dtype != GDR_FP32))
        return fail(GDR_ERR_INVALID_ARG, "unknown dtype (in %d, out %d)", d->in_dtype, d->out_dtype);
    if (!std::isfinite(d->scale)) return fail(GDR_ERR_INVALID_ARG, "scale is not finite");
    if (d->route != GDR_ROUTE_VALUE && d->route != GDR_ROUTE_ERROR)
        return fail(GDR_ERR_INVALID_ARG, "unknown epilogue route %d", d->route);
    if (d->prologue < GDR_PROLOGUE_NONE || d->prologue > GDR_PROLOGUE_ALPHA_FORGET)
        return fail(GDR_ERR_INVALID_ARG, "unknown prologue %d", d->prologue);
    if (d->dk != d->dv || (d->dk != 64 && d->dk != 128))
        return fail(GDR_ERR_UNSUPPORTED, "only dk == dv in {64, 128} is supported (got %lld, %lld)",
                    (long long)d->dk, (long long)d->dv);
    if (d->chunk != 0 && d->chunk != kChunk)
        return fail(GDR_ERR_UNSUPPORTED, "only chunk size 64 is supported (got %d)", d->chunk);
    // sizes: keep every element index and grid dimension in range
    const int64_t lim = int64_t(1) << 40;
    if (d->B > lim || d->T > lim || d->H > (int64_t(1) << 24))
        return fail(GDR_ERR_INVALID_ARG, "sizes out of range");
    const double elems = double(d->B) * double(d->T) * double(d->H) * double(d->dk);
    if (elems > 9.0e15) return fail(GDR_ERR_INVALID_ARG, "tensor too large");
    const int64_t nc = (d->T + kChunk - 1) / kChunk;
    const double blocks = double(d->B) * double(d->H) * double(nc > 0 ? nc : 1);
    const double state_blocks = double(d->B) * double(d->H) * double(d->dk / 16);
    if (blocks > 2147483647.0 || state_blocks > 2147483647.0)
        return fail(GDR_ERR_INVALID_ARG, "too many chunks for one launch");
    if (NC) *NC = nc;
    return GDR_OK;
}

// ---------------------------------------------------------------------------
// Debug mode (GDR_VALIDATE=1 in the environment, read at every call): after
// the host checks, every input tensor is checked on the device against the
// domain of the kernels (finite values; alpha in (0, 1]; for bf16 inputs the
// fp16 operand range) and the call synchronises the stream to read the result.
// A violation returns GDR_ERR_INVALID_ARG before any compute kernel is launched.
// ---------------------------------------------------------------------------
bool validate_on() {
    const char* e = std::getenv("GDR_VALIDATE");
    return e && e[0] == '1' && e[1] == '\0';
}

struct Check {
    const void* p;
    int64_t n;
    bool bf16;
    uint32_t rules;
    const char* name;
};

std::mutex g_check_mu;
unsigned long long* g_check_res[kMaxDevices] = {};

const char* rule_text(unsigned long long bits) {
    if (bits & gdr::CHECK_FINITE) return "is not finite (NaN or Inf)";
    if (bits & gdr::CHECK_ALPHA_OPEN) return "is outside (0, 1] (the chunked kernels take its logarithm)";
    if (bits & gdr::CHECK_ALPHA_CLOSED) return "is outside [0, 1]";
    if (bits & gdr::CHECK_NONZERO) return "is 0 (the error route divides the written update by beta)";
    if (bits & gdr::CHECK_FP16_RANGE)
        return "has magnitude >= 65504, beyond the fp16 operands that bf16 inputs are computed with";
    return "breaks an input rule";
}

gdr_status run_checks(const Check* c, int count, hipStream_t s) {
    if (!validate_on()) return GDR_OK;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess)
        return fail(GDR_ERR_DEVICE, "GDR_VALIDATE: cannot query the stream");
    if (cs != hipStreamCaptureStatusNone)
        return fail(GDR_ERR_INVALID_ARG, "GDR_VALIDATE=1 synchronises the stream; it cannot run under graph capture");
    std::lock_guard<std::mutex> lock(g_check_mu);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(GDR_ERR_DEVICE, "GDR_VALIDATE: no current device");
    if (!g_check_res[dev] && gdr::check_result_address(&g_check_res[dev]) != hipSuccess) {
        g_check_res[dev] = nullptr;
        return fail(GDR_ERR_DEVICE, "GDR_VALIDATE: check buffer unavailable");
    }
    for (int i = 0; i < count; ++i) {
        if (!c[i].p || c[i].n <= 0) continue;
        unsigned long long res[2] = {0, 0};
        if (gdr::launch_check(c[i].p, c[i].n, c[i].bf16, c[i].rules, g_check_res[dev], s) != hipSuccess ||
            hipMemcpyAsync(res, g_check_res[dev], sizeof res, hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
            return fail(GDR_ERR_DEVICE, "GDR_VALIDATE: check of %s failed to run", c[i].name);
        if (res[0])
            return fail(GDR_ERR_INVALID_ARG, "GDR_VALIDATE: %s[%llu] %s", c[i].name, res[1], rule_text(res[0]));
    }
    return GDR_OK;
}

// Epilogue scale gradient, reduced in two passes: CLVR sums token segments;
// the error-routing epilogue leaves one partial row per chunk.
int64_t dlam_segments(const gdr_desc* d) {
    const int64_t bt = d->B * d->T;
    return bt < 1 ? 1 : (bt < 256 ? bt : 256);
}
// fp32 [B, H, dk, dv]: the state (gradient) handed between the ranges of a cut pass
size_t carry_bytes(const gdr_desc* d) {
    return d->T > 0 ? size_t(d->B) * size_t(d->H) * size_t(d->dk) * size_t(d->dv) * 4 : 0;
}

size_t dlam_partial_bytes(const gdr_desc* d) {
    if (d->route == GDR_ROUTE_ERROR) {
        const int64_t nc = (d->T + kChunk - 1) / kChunk;
        return size_t(d->B) * size_t(nc) * size_t(d->H) * size_t(d->dv) * 4;
    }
    return size_t(dlam_segments(d)) * size_t(d->H) * size_t(d->dv) * 4;
}

}  // namespace

namespace gdr {

// Carves the chunk workspace; returns the bytes needed.  `base` may be NULL
// (sizing only).
size_t chunk_ws_bytes(int64_t nch, int D, int op_bytes, bool backward, bool cler, bool pro, ChunkWs* out,
                      void* base) {
    ChunkWs w;
    std::memset(&w, 0, sizeof w);
    size_t off = 0;
    char* p = static_cast<char*>(base);
    auto take = [&](size_t bytes) -> void* {
        void* r = p ? p + off : nullptr;
        off += align_up(bytes);
        return r;
    };
    const size_t mat = size_t(nch) * kChunk * D * op_bytes;    // [64][D] per chunk-head
    const size_t sq = size_t(nch) * kChunk * kChunk * op_bytes;  // [64][64]
    const size_t st = size_t(nch) * D * D * op_bytes;            // [D][D]
    w.W = take(mat);
    w.Ut = take(mat);
    w.Qt = take(mat);
    w.KbT = take(mat);
    w.A = take(sq);
    w.gam = static_cast<float*>(take(size_t(nch) * D * 4));
    // chunk-start states and U: written by the state pass, read by the output
    // kernel and the gradient kernels
    w.Ssnap = take(st);
    w.Usave = take(mat);
    if (pro) {
        // one float per token-head each (nch * 64 covers B * T * H)
        w.Bact = static_cast<float*>(take(size_t(nch) * kChunk * 4));
        w.rq = static_cast<float*>(take(size_t(nch) * kChunk * 4));
        w.rk = static_cast<float*>(take(size_t(nch) * kChunk * 4));
    }
    if (backward) {
        const size_t sq32 = size_t(nch) * kChunk * kChunk * 4;
        // fp32 operands: the transposes the reverse pass reads (with fp16 operands
        // it reads them from Qt, A, Kb^T and W with transposed LDS reads)
        if (op_bytes == 4) {
            w.AT = take(sq);
            w.Kb = take(mat);
            w.QtT = take(mat);
            w.WT = take(mat);
        }
        w.Nw = static_cast<float*>(take(sq32));
        w.Pw = static_cast<float*>(take(sq32));
        w.dSsnap = take(st);
        w.dUsave = take(mat);
        // fp16 operands: the gradient kernel reads dU's transpose from its LDS
        // copy of dU; fp32 operands keep the transposed copy
        if (op_bytes == 4) w.dUsaveT = take(mat);
        // the gradient partials the stages do not hand on chip
        const bool all = cler || grad_split(D, op_bytes == 4);
        if (all || !grad_qkb_on_chip(D)) {
            w.gQt = take(mat);
            w.gKb = take(mat);
        }
        if (all) {
            w.gKt = take(mat);
            w.gA = take(sq);
            w.gP = take(sq);
            w.gGam = static_cast<float*>(take(size_t(nch) * D * 4));
        }
        if (cler) w.Mt = take(mat);
    }
    if (out) *out = w;
    return off;
}

}  // namespace gdr

extern "C" {

const char* gdr_status_string(gdr_status s) {
    switch (s) {
        case GDR_OK: return "GDR_OK";
        case GDR_ERR_INVALID_ARG: return "GDR_ERR_INVALID_ARG";
        case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED";
        case GDR_ERR_WORKSPACE: return "GDR_ERR_WORKSPACE";
        case GDR_ERR_DEVICE: return "GDR_ERR_DEVICE";
    }
    return "GDR_ERR_UNKNOWN";
}

const char* gdr_last_error(void) { return g_err; }

int32_t gdr_version(void) { return 200; }

size_t gdr_workspace_size(const gdr_desc* desc, int op) {
    int64_t NC = 0;
    if (check_desc(desc, &NC) != GDR_OK) return 0;
    if (op != 0 && op != 1) {
        fail(GDR_ERR_INVALID_ARG, "op must be 0 (forward) or 1 (backward)");
        return 0;
    }
    const int64_t nch = desc->B * desc->H * NC;
    const int opb = desc->in_dtype == GDR_FP32 ? 4 : 2;
    size_t n = gdr::chunk_ws_bytes(nch, int(desc->dk), opb, op == 1, desc->route == GDR_ROUTE_ERROR,
                                   desc->prologue != GDR_PROLOGUE_NONE, nullptr, nullptr);
    if (op == 1) n += align_up(dlam_partial_bytes(desc));
    return n + align_up(carry_bytes(desc));
}

}  // extern "C"

// Forward.  train = true also keeps in ws everything the backward needs (the
// backward layout of the workspace), so that gdr_backward_saved can skip the
// recomputation.
static gdr_status forward_impl(const gdr_desc* desc, const void* q, const void* k, const void* v,
                               const float* beta, const float* alpha, const float* S0, void* o,
                               float* ST, void* h_clvr, const float* clvr_scale, void* ws,
                               size_t ws_bytes, void* stream, bool train, const void* gate_g = nullptr,
                               const float* gate_w = nullptr) {
    int64_t NC = 0;
    gdr_status st = check_desc(desc, &NC);
    if (st != GDR_OK) return st;
    const int64_t B = desc->B, T = desc->T, H = desc->H, D = desc->dk;
    const int64_t ntok = B * T * H;
    const bool any = ntok > 0;
    if (any && (!q || !k || !v || !beta || !o))
        return fail(GDR_ERR_INVALID_ARG, "q, k, v, beta and o are required");
    if ((desc->gate == GDR_GATE_NONE) != (alpha == nullptr) && any)
        return fail(GDR_ERR_INVALID_ARG, "alpha must be NULL iff the gate is NONE");
    if (any && gate_w && !gate_g) return fail(GDR_ERR_INVALID_ARG, "the output gate's w given without g");
    const void* ptrs[] = {q, k, v, beta, alpha, S0, o, ST, h_clvr, clvr_scale, ws, gate_g, gate_w};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(GDR_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
    if (clvr_scale && !h_clvr) return fail(GDR_ERR_INVALID_ARG, "clvr_scale given without h_clvr");
    const size_t ib = dtype_bytes(desc->in_dtype), ob = dtype_bytes(desc->out_dtype);
    const size_t n_in = size_t(ntok) * D;
    const size_t o_bytes = n_in * ob;
    const size_t a_bytes = desc->gate == GDR_GATE_CHANNEL ? n_in * 4 : size_t(ntok) * 4;
    const size_t s_bytes = size_t(B * H) * D * D * 4;
    struct {
        const void* p;
        size_t n;
    } ins[] = {{q, n_in * ib}, {k, n_in * ib}, {v, n_in * ib}, {beta, size_t(ntok) * 4},
               {alpha, a_bytes}, {S0, s_bytes}, {clvr_scale, size_t(H) * D * 4},
               {gate_g, n_in * ib}, {gate_w, size_t(H) * D * 4}};
    for (auto& in : ins) {
        if (overlap(o, o_bytes, in.p, in.n)) return fail(GDR_ERR_INVALID_ARG, "o overlaps an input");
        if (ST && in.p != S0 && overlap(ST, s_bytes, in.p, in.n))
            return fail(GDR_ERR_INVALID_ARG, "ST overlaps an input other than S0");
        if (h_clvr && in.p != nullptr && overlap(h_clvr, n_in * ib, in.p, in.n))
            return fail(GDR_ERR_INVALID_ARG, "h_clvr overlaps an input");
    }
    if (ST && overlap(ST, s_bytes, o, o_bytes)) return fail(GDR_ERR_INVALID_ARG, "ST overlaps o");
    if (h_clvr && overlap(h_clvr, n_in * ib, o, o_bytes))
        return fail(GDR_ERR_INVALID_ARG, "h_clvr overlaps o");
    if (S0 && ST && S0 != ST && overlap(S0, s_bytes, ST, s_bytes))
        return fail(GDR_ERR_INVALID_ARG, "ST partially overlaps S0 (it may only alias it exactly)");
    const int64_t nch = B * H * NC;
    const int opb = desc->in_dtype == GDR_FP32 ? 4 : 2;
    gdr::ChunkWs w;
    const int pro = desc->prologue;
    const size_t chunk_bytes =
        gdr::chunk_ws_bytes(nch, int(D), opb, train, desc->route == GDR_ROUTE_ERROR, pro != 0, &w, ws);
    const size_t need = (train ? chunk_bytes + align_up(dlam_partial_bytes(desc)) : chunk_bytes) +
                        align_up(carry_bytes(desc));
    if (ws_bytes < need || (need > 0 && !ws))
        return fail(GDR_ERR_WORKSPACE, "workspace too small: need %zu bytes, got %zu", need, ws_bytes);
    if (B * H == 0) return GDR_OK;
    if (ws) {
        for (auto& in : ins)
            if (overlap(ws, need, in.p, in.n)) return fail(GDR_ERR_INVALID_ARG, "workspace overlaps an input");
        if (overlap(ws, need, o, o_bytes) || (ST && overlap(ws, need, ST, s_bytes)) ||
            (h_clvr && overlap(ws, need, h_clvr, n_in * ib)))
            return fail(GDR_ERR_INVALID_ARG, "workspace overlaps an output");
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool in_f32 = desc->in_dtype == GDR_FP32, out_f32 = desc->out_dtype == GDR_FP32;
    {
        const bool bf = !in_f32;
        const int pro_ = desc->prologue;
        const uint32_t F = gdr::CHECK_FINITE, R = bf ? gdr::CHECK_FP16_RANGE : 0u;
        const uint32_t beta_rules =
            F | ((h_clvr && desc->route == GDR_ROUTE_ERROR && !pro_) ? gdr::CHECK_NONZERO : 0u);
        const Check checks[] = {
            {q, int64_t(n_in), bf, F | (pro_ ? 0u : R), "q"},
            {k, int64_t(n_in), bf, F | (pro_ ? 0u : R), "k"},
            {v, int64_t(n_in), bf, F | R, "v"},
            {beta, ntok, false, beta_rules, "beta"},
            {alpha, int64_t(a_bytes / 4), false, pro_ ? F : gdr::CHECK_ALPHA_OPEN, "alpha"},
            {S0, int64_t(s_bytes / 4), false, F | R, "S0"},
            {h_clvr, int64_t(n_in), bf, F, "h_clvr"},
            {clvr_scale, H * D, false, F, "clvr_scale"},
            {gate_g, int64_t(n_in), bf, F, "g"},
            {gate_w, H * D, false, F, "w"},
        };
        gdr_status g = run_checks(checks, int(sizeof checks / sizeof checks[0]), s);
        if (g != GDR_OK) return g;
    }
    // the value-routing epilogue runs in the intra-chunk kernel (it needs only
    // v); the error-routing one needs U, so it follows the state pass
    const bool cler = h_clvr && desc->route == GDR_ROUTE_ERROR;
    // with the prologue the kernels after the intra-chunk one read its activated beta
    const float* beta_eff = pro ? w.Bact : beta;
    hipError_t e = hipSuccess;
    auto intra = [&](gdr::ChunkRange cr, hipStream_t is) -> gdr_status {
        gdr::prof_before(is);
        e = gdr::launch_intra(int(D), desc->gate, in_f32, train ? 2 : 0, B, T, int(H), NC, q, k, v, beta,
                              alpha, cler ? nullptr : h_clvr, cler ? nullptr : clvr_scale, w, pro, cr, is);
        gdr::prof_after(train ? "intra_train" : "intra_fwd", is);
        if (e != hipSuccess) return fail(GDR_ERR_DEVICE, "intra-chunk launch: %s", hipGetErrorString(e));
        return GDR_OK;
    };
    const char* st_name = train ? "state_train" : "state_fwd";
    const char* out_name = gate_g ? "output_gated" : cler ? "output_cler" : "output";
    const gdr::OutGate og{gate_g, gate_w};
    auto output = [&](gdr::ChunkRange cr, hipStream_t os) -> gdr_status {
        gdr::prof_before(os);
        e = gate_g ? gdr::launch_output_gated(int(D), out_f32, B, T, int(H), NC, desc->scale, w, o, beta_eff,
                                              clvr_scale, cler ? h_clvr : nullptr, og, cr, os)
                   : gdr::launch_output(int(D), out_f32, B, T, int(H), NC, desc->scale, w, o, beta_eff, clvr_scale,
                                        cler ? h_clvr : nullptr, cr, os);
        gdr::prof_after(out_name, os);
        if (e != hipSuccess) return fail(GDR_ERR_DEVICE, "output launch: %s", hipGetErrorString(e));
        return GDR_OK;
    };
    // two state slices per workgroup when the chain has more slices than there are CUs
    bool wide = false;
    {
        std::lock_guard<std::mutex> lock(g_aux_mu);
        Aux* aux = (!in_f32 && NC > 0) ? aux_stream() : nullptr;
        const int parts = state_parts(aux, B * H * (D / 16), NC);
        wide = aux && B * H * (D / 16) > aux->cus;
        if (parts > 1) {
            // The chain in `parts` ranges (state handed through the workspace).
            // Range p's intra-chunk transform runs on the second stream while
            // the chain carries range p-1 (the chain holds only part of the chip),
            // and the output of each finished range on the third.  Events: ev[p]
            // intra range p done, ev[parts + p] chain range p done.  The first
            // chain range, beside most of the intra-chunk work, carries two
            // slices per workgroup to leave that work more CUs; the later ones
            // one (at the 32K-token KDA shape: inference forward 0.951 ms,
            // against 0.960 with one slice and 0.985 with two throughout; the
            // two-slice chain steps slower beside the intra-chunk kernel).
            float* carry = reinterpret_cast<float*>(static_cast<char*>(ws) + need - align_up(carry_bytes(desc)));
            int64_t lo[kMaxParts], hi[kMaxParts];
            for (int p = 0; p < parts; ++p) cut_range(NC, parts, p, false, &lo[p], &hi[p], train ? 3 : 4, train ? 2 : 3);
            gdr_status g = intra(gdr::ChunkRange{lo[0], hi[0] - lo[0]}, s);
            if (g != GDR_OK) return g;
            if (hipEventRecord(aux->ev[0], s) != hipSuccess || hipStreamWaitEvent(aux->s, aux->ev[0], 0) != hipSuccess)
                return fail(GDR_ERR_DEVICE, "stream ordering failed");
            for (int p = 1; p < parts; ++p) {
                g = intra(gdr::ChunkRange{lo[p], hi[p] - lo[p]}, aux->s);
                if (g != GDR_OK) return g;
                if (hipEventRecord(aux->ev[p], aux->s) != hipSuccess)
                    return fail(GDR_ERR_DEVICE, "stream ordering failed");
            }
            for (int p = 0; p < parts; ++p) {
                if (p > 0 && hipStreamWaitEvent(s, aux->ev[p], 0) != hipSuccess)
                    return fail(GDR_ERR_DEVICE, "stream ordering failed");
                gdr::prof_before(s);
                e = gdr::launch_state_fwd(int(D), in_f32, out_f32, B, T, int(H), NC, desc->scale, w,
                                          p == 0 ? S0 : carry, p == parts - 1 ? ST : carry, o, true,
                                          p == 0, gdr::ChunkRange{lo[p], hi[p] - lo[p]}, s);
                gdr::prof_after(st_name, s);
                if (e != hipSuccess) return fail(GDR_ERR_DEVICE, "state-pass launch: %s", hipGetErrorString(e));
                if (hipEventRecord(aux->ev[parts + p], s) != hipSuccess ||
                    hipStreamWaitEvent(aux->s2, aux->ev[parts + p], 0) != hipSuccess)
                    return fail(GDR_ERR_DEVICE, "stream ordering failed");
                g = output(gdr::ChunkRange{lo[p], hi[p] - lo[p]}, aux->s2);
                if (g != GDR_OK) return g;
            }
            // the second stream's last work (intra of the last range) is ordered
            // before the last chain range; the third stream rejoins here
            if (hipEventRecord(aux->ev[kAuxEvents - 1], aux->s2) != hipSuccess ||
                hipStreamWaitEvent(s, aux->ev[kAuxEvents - 1], 0) != hipSuccess)
                return fail(GDR_ERR_DEVICE, "stream ordering failed");
            return GDR_OK;
        }
    }
    if (NC > 0) {
        gdr_status g = intra(gdr::ChunkRange{0, NC}, s);
        if (g != GDR_OK) return g;
    }
    gdr::prof_before(s);
    e = gdr::launch_state_fwd(int(D), in_f32, out_f32, B, T, int(H), NC, desc->scale, w, S0, ST, o,
                              train || cler, wide, gdr::ChunkRange{0, NC}, s);
    gdr::prof_after(st_name, s);
    if (e != hipSuccess) return fail(GDR_ERR_DEVICE, "state-pass launch: %s", hipGetErrorString(e));
    if (!in_f32 && NC > 0) {
        gdr_status g = output(gdr::ChunkRange{0, NC}, s);
        if (g != GDR_OK) return g;
    }
    if (in_f32 && cler && NC > 0) {
        gdr::prof_before(s);
        e = gdr::launch_cler_fwd(int(D), in_f32, B, T, int(H), NC, w, beta_eff, clvr_scale, h_clvr, s);
        gdr::prof_after("cler_fwd", s);
        if (e != hipSuccess) return fail(GDR_ERR_DEVICE, "error-routing launch: %s", hipGetErrorString(e));
    }
    if (in_f32 && gate_g) {
        // fp32 operands: the state pass writes o, and the gate runs over it in place
        gdr::prof_before(s);
        e = gdr::launch_gate(false, int(D), true, out_f32, B * T, int(H), o, gate_g, gate_w, o, nullptr, nullptr,
                             nullptr, nullptr, nullptr, s);
        gdr::prof_after("gate_fwd", s);
        if (e != hipSuccess) return fail(GDR_ERR_DEVICE, "output-gate launch: %s", hipGetErrorString(e));
    }
    return GDR_OK;
}

// Backward.  recompute = false takes the forward's intermediates from ws, where
// a preceding forward_impl(train = true) with the same arguments left them.
static gdr_status backward_impl(const gdr_desc* desc, const void* q, const void* k, const void* v,
                                const float* beta, const float* alpha, const float* S0, const void* dO,
                                const float* dST, const void* dh_clvr, const float* clvr_scale, void* dq,
                                void* dk, void* dv, float* dbeta, float* dalpha, float* dS0,
                                float* dclvr_scale, void* ws, size_t ws_bytes, void* stream,
                                bool recompute) {
    int64_t NC = 0;
    gdr_status st = check_desc(desc, &NC);
    if (st != GDR_OK) return st;
    const int64_t B = desc->B, T = desc->T, H = desc->H, D = desc->dk;
    const int64_t ntok = B * T * H;
    const bool any = ntok > 0;
    if (any && (!q || !k || !v || !beta || !dO || !dq || !dk || !dv || !dbeta))
        return fail(GDR_ERR_INVALID_ARG, "q, k, v, beta, dO, dq, dk, dv and dbeta are required");
    if ((desc->gate == GDR_GATE_NONE) != (alpha == nullptr) && any)
        return fail(GDR_ERR_INVALID_ARG, "alpha must be NULL iff the gate is NONE");
    if ((desc->gate == GDR_GATE_NONE) != (dalpha == nullptr) && any)
        return fail(GDR_ERR_INVALID_ARG, "dalpha must be NULL iff the gate is NONE");
    if ((clvr_scale || dclvr_scale) && !dh_clvr)
        return fail(GDR_ERR_INVALID_ARG, "clvr_scale / dclvr_scale given without dh_clvr");
    const void* ptrs[] = {q, k, v, beta, alpha, S0, dO, dST, dh_clvr, clvr_scale, dq, dk, dv, dbeta,
                          dalpha, dS0, dclvr_scale, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(GDR_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
    const size_t ib = dtype_bytes(desc->in_dtype), ob = dtype_bytes(desc->out_dtype);
    const size_t n_in = size_t(ntok) * D;
    const size_t a_bytes = desc->gate == GDR_GATE_CHANNEL ? n_in * 4 : size_t(ntok) * 4;
    const size_t s_bytes = size_t(B * H) * D * D * 4;
    struct {
        const void* p;
        size_t n;
    } ins[] = {{q, n_in * ib}, {k, n_in * ib}, {v, n_in * ib}, {beta, size_t(ntok) * 4}, {alpha, a_bytes},
               {S0, s_bytes}, {dO, n_in * ib}, {dST, s_bytes}, {dh_clvr, n_in * ib},
               {clvr_scale, size_t(H) * D * 4}},
      outs[] = {{dq, n_in * ob}, {dk, n_in * ob}, {dv, n_in * ob}, {dbeta, size_t(ntok) * 4},
                {dalpha, a_bytes}, {dS0, s_bytes}, {dclvr_scale, size_t(H) * D * 4}};
    for (auto& o1 : outs) {
        for (auto& in : ins)
            if (overlap(o1.p, o1.n, in.p, in.n)) return fail(GDR_ERR_INVALID_ARG, "an output overlaps an input");
        for (auto& o2 : outs)
            if (&o1 != &o2 && overlap(o1.p, o1.n, o2.p, o2.n))
                return fail(GDR_ERR_INVALID_ARG, "two outputs overlap");
    }
    const int64_t nch = B * H * NC;
    const int opb = desc->in_dtype == GDR_FP32 ? 4 : 2;
    gdr::ChunkWs w;
    const int pro = desc->prologue;
    const size_t chunk_bytes =
        gdr::chunk_ws_bytes(nch, int(D), opb, true, desc->route == GDR_ROUTE_ERROR, pro != 0, &w, ws);
    const size_t need = chunk_bytes + align_up(dlam_partial_bytes(desc)) + align_up(carry_bytes(desc));
    if (ws_bytes < need || (need > 0 && !ws))
        return fail(GDR_ERR_WORKSPACE, "workspace too small: need %zu bytes, got %zu", need, ws_bytes);
    for (auto& o1 : outs)
        if (ws && overlap(ws, need, o1.p, o1.n)) return fail(GDR_ERR_INVALID_ARG, "workspace overlaps an output");
    for (auto& in : ins)
        if (ws && overlap(ws, need, in.p, in.n)) return fail(GDR_ERR_INVALID_ARG, "workspace overlaps an input");
    if (B * H == 0) return GDR_OK;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool in_f32 = desc->in_dtype == GDR_FP32, out_f32 = desc->out_dtype == GDR_FP32;
    const int gate = desc->gate;
    {
        const bool bf = !in_f32;
        const uint32_t F = gdr::CHECK_FINITE, R = bf ? gdr::CHECK_FP16_RANGE : 0u;
        const uint32_t beta_rules =
            F | ((dh_clvr && desc->route == GDR_ROUTE_ERROR && !pro) ? gdr::CHECK_NONZERO : 0u);
        const Check checks[] = {
            {q, int64_t(n_in), bf, F | (pro ? 0u : R), "q"},
            {k, int64_t(n_in), bf, F | (pro ? 0u : R), "k"},
            {v, int64_t(n_in), bf, F | R, "v"},
            {beta, ntok, false, beta_rules, "beta"},
            {alpha, int64_t(a_bytes / 4), false, pro ? F : gdr::CHECK_ALPHA_OPEN, "alpha"},
            {S0, int64_t(s_bytes / 4), false, F | R, "S0"},
            {dO, int64_t(n_in), bf, F | R, "dO"},
            {dST, int64_t(s_bytes / 4), false, F | R, "dST"},
            {dh_clvr, int64_t(n_in), bf, F | R, "dh_clvr"},
            {clvr_scale, H * D, false, F, "clvr_scale"},
        };
        gdr_status g = run_checks(checks, int(sizeof checks / sizeof checks[0]), s);
        if (g != GDR_OK) return g;
    }
    hipError_t e = hipSuccess;
#define GDR_STEP_ON(st, name, call)                                                           \
    do {                                                                                      \
        gdr::prof_before(st);                                                                 \
        e = (call);                                                                           \
        gdr::prof_after(name, st);                                                            \
        if (e != hipSuccess) return fail(GDR_ERR_DEVICE, "%s launch: %s", name, hipGetErrorString(e)); \
    } while (0)
#define GDR_STEP(name, call) GDR_STEP_ON(s, name, call)
    if (NC > 0 && recompute) {
        GDR_STEP("intra_bwd", gdr::launch_intra(int(D), gate, in_f32, 1, B, T, int(H), NC, q, k, v, beta,
                                                alpha, nullptr, nullptr, w, pro, gdr::ChunkRange{0, NC}, s));
        bool wide = false;
        if (!in_f32) {
            std::lock_guard<std::mutex> lock(g_aux_mu);
            const Aux* aux = aux_stream();
            wide = aux && B * H * (D / 16) > aux->cus;
        }
        GDR_STEP("state_fwd_save", gdr::launch_state_fwd(int(D), in_f32, out_f32, B, T, int(H), NC,
                                                         desc->scale, w, S0, nullptr, nullptr, true, wide,
                                                         gdr::ChunkRange{0, NC}, s));
    }
    // error routing: dh reaches U inside the reverse state pass and beta and the
    // scale afterwards; value routing: dh reaches v in the gradient kernel
    const bool cler = dh_clvr && desc->route == GDR_ROUTE_ERROR;
    // with the prologue the kernels after the intra-chunk one read its activated beta
    const float* beta_eff = pro ? w.Bact : beta;
    if (cler && NC > 0)
        GDR_STEP("cler_mt", gdr::launch_cler_mt(int(D), in_f32, B, T, int(H), NC, w, clvr_scale, dh_clvr, s));
    float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + chunk_bytes);
    float* carry =
        reinterpret_cast<float*>(static_cast<char*>(ws) + chunk_bytes + align_up(dlam_partial_bytes(desc)));
    // per-chunk gradient kernels of one chunk range, on stream `gs` (ahead: see
    // grads_ahead)
    auto grads = [&](gdr::ChunkRange cr, hipStream_t gs, int ahead) -> gdr_status {
        // both routes add lam * dh to dv: the value route through v itself, the
        // error route through e = v - ...; the error route's own terms run
        // between the two gradient stages, in the same kernel
        GDR_STEP_ON(gs, cler ? "grads_cler" : "grads",
                    gdr::launch_grads(int(D), gate, in_f32, out_f32, B, T, int(H), NC, desc->scale, q, k, v, beta_eff,
                                      alpha, dO, dh_clvr, clvr_scale, dq, dk, dv, dbeta, dalpha, w, pro, cr, cler,
                                      cler && dclvr_scale ? partial : nullptr, ahead, gs));
        return GDR_OK;
    };
    const char* sb_name = cler ? "state_bwd_cler" : "state_bwd";
    const void* dh_state = cler ? dh_clvr : nullptr;
    {
        std::lock_guard<std::mutex> lock(g_aux_mu);
        Aux* aux = NC > 0 ? aux_stream() : nullptr;
        const int parts = state_parts(aux, B * H * (D / 16), NC);
        // two state slices per workgroup when the pass shares the chip with the
        // gradient kernels or has more slices than there are CUs
        const bool wide = parts > 1 || (aux && B * H * (D / 16) > aux->cus);
        if (parts == 1) {
            GDR_STEP(sb_name, gdr::launch_state_bwd(int(D), in_f32, B, T, int(H), NC, desc->scale, w, dO, dST, dS0,
                                                    dh_state, clvr_scale, beta_eff, wide, gdr::ChunkRange{0, NC}, s));
            if (NC > 0) {
                gdr_status g = grads(gdr::ChunkRange{0, NC}, s, grads_ahead(aux, 0));
                if (g != GDR_OK) return g;
            }
        } else {
            // reverse pass in `parts` ranges, last chunks first; the gradient
            // kernels of each finished range run on the second stream.  Nothing
            // runs beside the first range, so it keeps one slice per workgroup
            // (its faster step; 2.63 against 2.645 ms per training step at the
            // 32K-token KDA shape)
            for (int p = 0; p < parts; ++p) {
                int64_t lo, hi;
                cut_range(NC, parts, p, true, &lo, &hi, 3, 2);
                GDR_STEP(sb_name, gdr::launch_state_bwd(int(D), in_f32, B, T, int(H), NC, desc->scale, w, dO,
                                                        p == 0 ? dST : carry, p == parts - 1 ? dS0 : carry,
                                                        dh_state, clvr_scale, beta_eff, wide && p > 0,
                                                        gdr::ChunkRange{lo, hi - lo}, s));
                if (hipEventRecord(aux->ev[p], s) != hipSuccess || hipStreamWaitEvent(aux->s, aux->ev[p], 0) != hipSuccess)
                    return fail(GDR_ERR_DEVICE, "stream ordering failed");
                // the next range of the reverse pass holds one CU per workgroup
                const int64_t busy = p + 1 < parts ? B * H * (D / 16) / (wide ? 2 : 1) : 0;
                gdr_status g = grads(gdr::ChunkRange{lo, hi - lo}, aux->s, grads_ahead(aux, busy));
                if (g != GDR_OK) return g;
            }
            // the value-route scale gradient needs only dh and v: it runs on the
            // caller's stream beside the last range's gradient kernels (at the
            // 32K-token KDA shape 2.65 ms per training step, against 2.68 beside
            // the first range of the reverse pass, where it delays the first
            // gradient kernels)
            if (!cler && dclvr_scale)
                GDR_STEP("clvr_dlam", gdr::launch_clvr_dlam(in_f32, B * T, int(H), int(D), dh_clvr, v, dclvr_scale,
                                                            partial, dlam_segments(desc), s));
            if (hipEventRecord(aux->ev[kAuxEvents - 1], aux->s) != hipSuccess ||
                hipStreamWaitEvent(s, aux->ev[kAuxEvents - 1], 0) != hipSuccess)
                return fail(GDR_ERR_DEVICE, "stream ordering failed");
            if (cler && dclvr_scale)
                GDR_STEP("cler_dlam", gdr::launch_dlam_final(int(H * D), B * NC, partial, dclvr_scale, s));
            return GDR_OK;
        }
    }
    if (cler) {
        if (dclvr_scale) GDR_STEP("cler_dlam", gdr::launch_dlam_final(int(H * D), B * NC, partial, dclvr_scale, s));
    } else if (dclvr_scale) {
        GDR_STEP("clvr_dlam", gdr::launch_clvr_dlam(in_f32, B * T, int(H), int(D), dh_clvr, v, dclvr_scale,
                                                    partial, dlam_segments(desc), s));
    }
#undef GDR_STEP
#undef GDR_STEP_ON
    return GDR_OK;
}

// ---------------------------------------------------------------------------
// Gated DeltaNet-2 (separate erase and write gates): fp32 chunk operands and the
// two additive terms X, Y per chunk-head.
// ---------------------------------------------------------------------------
static size_t gdn2_ws_bytes(int64_t nch, int D, int op_bytes, gdr::ChunkWs* out, void* base) {
    gdr::ChunkWs w;
    std::memset(&w, 0, sizeof w);
    size_t off = 0;
    char* p = static_cast<char*>(base);
    auto take = [&](size_t bytes) -> void* {
        void* r = p ? p + off : nullptr;
        off += align_up(bytes);
        return r;
    };
    const size_t mat = size_t(nch) * kChunk * D * op_bytes;  // [64][D] in operand precision
    w.W = take(mat);
    w.Ut = take(mat);
    w.Qt = take(mat);
    w.KbT = take(mat);
    w.A = take(size_t(nch) * kChunk * kChunk * op_bytes);
    w.gam = static_cast<float*>(take(size_t(nch) * D * 4));
    w.X = static_cast<float*>(take(size_t(nch) * D * D * 4));       // fp32
    w.Y = static_cast<float*>(take(size_t(nch) * kChunk * D * 4));  // fp32
    if (out) *out = w;
    return off;
}

// The separate-gate workspace plus the fp32 state handed between the ranges of
// a cut pass (at the end, as in the chunked forward's).
static size_t gdn2_ws_total(const gdr_desc* d, int64_t NC) {
    return gdn2_ws_bytes(d->B * d->H * NC, int(d->dk), d->in_dtype == GDR_FP32 ? 4 : 2, nullptr, nullptr) +
           align_up(carry_bytes(d));
}

static gdr_status gdn2_check_desc(const gdr_desc* desc, int64_t* NC) {
    gdr_status st = check_desc(desc, NC);
    if (st != GDR_OK) return st;
    if (desc->route != GDR_ROUTE_VALUE || desc->prologue != GDR_PROLOGUE_NONE)
        return fail(GDR_ERR_UNSUPPORTED, "the separate-gate variant takes no hidden-stream route and no prologue");
    return GDR_OK;
}

extern "C" size_t gdr_gdn2_workspace_size(const gdr_desc* desc) {
    int64_t NC = 0;
    if (gdn2_check_desc(desc, &NC) != GDR_OK) return 0;
    return gdn2_ws_total(desc, NC);
}

extern "C" gdr_status gdr_gdn2_forward_chunked(const gdr_desc* desc, const void* q, const void* k, const void* v,
                                               const float* erase, const float* write, const float* alpha,
                                               const float* S0, void* o, float* ST, void* ws, size_t ws_bytes,
                                               void* stream) {
    int64_t NC = 0;
    gdr_status st = gdn2_check_desc(desc, &NC);
    if (st != GDR_OK) return st;
    const int64_t B = desc->B, T = desc->T, H = desc->H, D = desc->dk;
    const int64_t ntok = B * T * H;
    const bool any = ntok > 0;
    if (any && (!q || !k || !v || !erase || !write || !o))
        return fail(GDR_ERR_INVALID_ARG, "q, k, v, erase, write and o are required");
    if ((desc->gate == GDR_GATE_NONE) != (alpha == nullptr) && any)
        return fail(GDR_ERR_INVALID_ARG, "alpha must be NULL iff the gate is NONE");
    const void* ptrs[] = {q, k, v, erase, write, alpha, S0, o, ST, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(GDR_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
    const size_t ib = dtype_bytes(desc->in_dtype), ob = dtype_bytes(desc->out_dtype);
    const size_t n_in = size_t(ntok) * D;
    const size_t o_bytes = n_in * ob;
    const size_t a_bytes = desc->gate == GDR_GATE_CHANNEL ? n_in * 4 : size_t(ntok) * 4;
    const size_t s_bytes = size_t(B * H) * D * D * 4;
    struct {
        const void* p;
        size_t n;
    } ins[] = {{q, n_in * ib}, {k, n_in * ib}, {v, n_in * ib}, {erase, n_in * 4}, {write, n_in * 4},
               {alpha, a_bytes}, {S0, s_bytes}};
    for (auto& in : ins) {
        if (overlap(o, o_bytes, in.p, in.n)) return fail(GDR_ERR_INVALID_ARG, "o overlaps an input");
        if (ST && in.p != S0 && overlap(ST, s_bytes, in.p, in.n))
            return fail(GDR_ERR_INVALID_ARG, "ST overlaps an input other than S0");
    }
    if (ST && overlap(ST, s_bytes, o, o_bytes)) return fail(GDR_ERR_INVALID_ARG, "ST overlaps o");
    if (S0 && ST && S0 != ST && overlap(S0, s_bytes, ST, s_bytes))
        return fail(GDR_ERR_INVALID_ARG, "ST partially overlaps S0 (it may only alias it exactly)");
    gdr::ChunkWs w;
    gdn2_ws_bytes(B * H * NC, int(D), desc->in_dtype == GDR_FP32 ? 4 : 2, &w, ws);
    const size_t need = gdn2_ws_total(desc, NC);
    if (ws_bytes < need || (need > 0 && !ws))
        return fail(GDR_ERR_WORKSPACE, "workspace too small: need %zu bytes, got %zu", need, ws_bytes);
    if (B * H == 0) return GDR_OK;
    if (ws) {
        for (auto& in : ins)
            if (overlap(ws, need, in.p, in.n)) return fail(GDR_ERR_INVALID_ARG, "workspace overlaps an input");
        if (overlap(ws, need, o, o_bytes) || (ST && overlap(ws, need, ST, s_bytes)))
            return fail(GDR_ERR_INVALID_ARG, "workspace overlaps an output");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool in_f32 = desc->in_dtype == GDR_FP32, out_f32 = desc->out_dtype == GDR_FP32;
    {
        const uint32_t F = gdr::CHECK_FINITE, R = in_f32 ? 0u : gdr::CHECK_FP16_RANGE;
        const Check checks[] = {
            {q, int64_t(n_in), !in_f32, F, "q"},         {k, int64_t(n_in), !in_f32, F, "k"},
            {v, int64_t(n_in), !in_f32, F | R, "v"},     {erase, int64_t(n_in), false, F, "erase"},
            {write, int64_t(n_in), false, F, "write"},   {alpha, int64_t(a_bytes / 4), false, gdr::CHECK_ALPHA_OPEN, "alpha"},
            {S0, int64_t(s_bytes / 4), false, F, "S0"},
        };
        gdr_status g = run_checks(checks, int(sizeof checks / sizeof checks[0]), s);
        if (g != GDR_OK) return g;
    }
    hipError_t e = hipSuccess;
    auto intra = [&](gdr::ChunkRange cr, hipStream_t is) -> gdr_status {
        gdr::prof_before(is);
        e = gdr::launch_gdn2_intra(int(D), desc->gate, in_f32, B, T, int(H), NC, q, k, v, erase, write, alpha, w,
                                   cr, is);
        gdr::prof_after("gdn2_intra", is);
        if (e != hipSuccess) return fail(GDR_ERR_DEVICE, "intra-chunk launch: %s", hipGetErrorString(e));
        return GDR_OK;
    };
    auto pass = [&](gdr::ChunkRange cr, const float* sin, float* sout) -> gdr_status {
        gdr::prof_before(s);
        e = gdr::launch_state_fwd_xy(int(D), in_f32, out_f32, B, T, int(H), NC, desc->scale, w, sin, sout, o, cr, s);
        gdr::prof_after("gdn2_state", s);
        if (e != hipSuccess) return fail(GDR_ERR_DEVICE, "state-pass launch: %s", hipGetErrorString(e));
        return GDR_OK;
    };
    {
        // As in the chunked forward: when the pass (one workgroup per 16-column
        // slice) leaves CUs idle, it is cut into chunk ranges, largest first, and
        // the intra-chunk transform of range p runs on the second stream while
        // the pass carries range p-1 (the output is computed in the pass).  At
        // B=1 H=16 T=32768 d=128: forward 1.27 ms uncut, 1.13 ms cut with range
        // ratio 5/4 (4/3: 1.13, 3/2: 1.14, 2: 1.17, 3: 1.21, equal ranges 1.17).
        std::lock_guard<std::mutex> lock(g_aux_mu);
        Aux* aux = (!in_f32 && NC > 0) ? aux_stream() : nullptr;
        const int parts = state_parts(aux, B * H * (D / 16), NC);
        if (parts > 1) {
            float* carry = reinterpret_cast<float*>(static_cast<char*>(ws) + need - align_up(carry_bytes(desc)));
            int64_t lo[kMaxParts], hi[kMaxParts];
            for (int p = 0; p < parts; ++p) cut_range(NC, parts, p, false, &lo[p], &hi[p], 5, 4);
            gdr_status g = intra(gdr::ChunkRange{lo[0], hi[0] - lo[0]}, s);
            if (g != GDR_OK) return g;
            if (hipEventRecord(aux->ev[0], s) != hipSuccess || hipStreamWaitEvent(aux->s, aux->ev[0], 0) != hipSuccess)
                return fail(GDR_ERR_DEVICE, "stream ordering failed");
            for (int p = 1; p < parts; ++p) {
                g = intra(gdr::ChunkRange{lo[p], hi[p] - lo[p]}, aux->s);
                if (g != GDR_OK) return g;
                if (hipEventRecord(aux->ev[p], aux->s) != hipSuccess)
                    return fail(GDR_ERR_DEVICE, "stream ordering failed");
            }
            // range p's pass waits for its intra-chunk range; the last wait also
            // orders all of the second stream's work before the caller's stream
            for (int p = 0; p < parts; ++p) {
                if (p > 0 && hipStreamWaitEvent(s, aux->ev[p], 0) != hipSuccess)
                    return fail(GDR_ERR_DEVICE, "stream ordering failed");
                g = pass(gdr::ChunkRange{lo[p], hi[p] - lo[p]}, p == 0 ? S0 : carry, p == parts - 1 ? ST : carry);
                if (g != GDR_OK) return g;
            }
            return GDR_OK;
        }
    }
    if (NC > 0) {
        gdr_status g = intra(gdr::ChunkRange{0, NC}, s);
        if (g != GDR_OK) return g;
    }
    return pass(gdr::ChunkRange{0, NC}, S0, ST);
}

extern "C" gdr_status gdr_gdn2_decode_step(int64_t N, int64_t H, int64_t dk, int64_t dv, int32_t gate,
                                           int32_t in_dtype, int32_t out_dtype, float scale, const void* q,
                                           const void* k, const void* v, const float* erase, const float* write,
                                           const float* alpha, float* S, void* o, void* stream) {
    gdr_desc d;
    std::memset(&d, 0, sizeof d);
    d.B = N; d.T = 1; d.H = H; d.dk = dk; d.dv = dv; d.gate = gate; d.in_dtype = in_dtype;
    d.out_dtype = out_dtype; d.scale = scale; d.chunk = 0;
    gdr_status st = check_desc(&d, nullptr);
    if (st != GDR_OK) return st;
    const int64_t nslab = N * H;
    if (nslab == 0) return GDR_OK;
    if (nslab > 2147483647LL) return fail(GDR_ERR_INVALID_ARG, "N*H too large for one launch");
    if (!q || !k || !v || !erase || !write || !S || !o)
        return fail(GDR_ERR_INVALID_ARG, "q, k, v, erase, write, S and o are required");
    if ((gate == GDR_GATE_NONE) != (alpha == nullptr))
        return fail(GDR_ERR_INVALID_ARG, "alpha must be NULL iff the gate is NONE");
    const void* ptrs[] = {q, k, v, erase, write, alpha, S, o};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(GDR_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
    const size_t ib = dtype_bytes(in_dtype), ob = dtype_bytes(out_dtype);
    const size_t n = size_t(nslab) * dk;
    const size_t s_bytes = size_t(nslab) * dk * dv * 4;
    const size_t a_bytes = gate == GDR_GATE_CHANNEL ? n * 4 : size_t(nslab) * 4;
    struct {
        const void* p;
        size_t n;
    } ins[] = {{q, n * ib}, {k, n * ib}, {v, n * ib}, {erase, n * 4}, {write, n * 4}, {alpha, a_bytes}};
    for (auto& in : ins) {
        if (overlap(o, n * ob, in.p, in.n)) return fail(GDR_ERR_INVALID_ARG, "o overlaps an input");
        if (overlap(S, s_bytes, in.p, in.n)) return fail(GDR_ERR_INVALID_ARG, "S overlaps an input");
    }
    if (overlap(S, s_bytes, o, n * ob)) return fail(GDR_ERR_INVALID_ARG, "o overlaps S");
    hipStream_t s = static_cast<hipStream_t>(stream);
    {
        const bool bf = in_dtype != GDR_FP32;
        const uint32_t F = gdr::CHECK_FINITE;
        const Check checks[] = {
            {q, int64_t(n), bf, F, "q"},         {k, int64_t(n), bf, F, "k"},         {v, int64_t(n), bf, F, "v"},
            {erase, int64_t(n), false, F, "erase"}, {write, int64_t(n), false, F, "write"},
            {alpha, int64_t(a_bytes / 4), false, gdr::CHECK_ALPHA_CLOSED, "alpha"},
            {S, int64_t(s_bytes / 4), false, F, "S"},
        };
        gdr_status g = run_checks(checks, int(sizeof checks / sizeof checks[0]), s);
        if (g != GDR_OK) return g;
    }
    gdr::prof_before(s);
    hipError_t e = gdr::launch_gdn2_decode(int(dk), gate, in_dtype == GDR_FP32, out_dtype == GDR_FP32, nslab, scale,
                                           q, k, v, erase, write, alpha, S, o, s);
    gdr::prof_after("gdn2_decode", s);
    if (e != hipSuccess) return fail(GDR_ERR_DEVICE, "decode launch: %s", hipGetErrorString(e));
    return GDR_OK;
}

namespace gdr {

// Entry points defined in other sources share the forward and the error text.
gdr_status forward_entry(const gdr_desc* desc, const void* q, const void* k, const void* v, const float* beta,
                         const float* alpha, const float* S0, void* o, float* ST, void* h_clvr,
                         const float* clvr_scale, void* ws, size_t ws_bytes, void* stream) {
    return forward_impl(desc, q, k, v, beta, alpha, S0, o, ST, h_clvr, clvr_scale, ws, ws_bytes, stream, false);
}

gdr_status set_error(gdr_status s, const char* msg) { return fail(s, "%s", msg); }

}  // namespace gdr

extern "C" {

gdr_status gdr_forward_chunked(const gdr_desc* desc, const void* q, const void* k, const void* v,
                               const float* beta, const float* alpha, const float* S0, void* o,
                               float* ST, void* h_clvr, const float* clvr_scale, void* ws,
                               size_t ws_bytes, void* stream) {
    return forward_impl(desc, q, k, v, beta, alpha, S0, o, ST, h_clvr, clvr_scale, ws, ws_bytes, stream, false);
}

gdr_status gdr_forward_chunked_gated(const gdr_desc* desc, const void* q, const void* k, const void* v,
                                     const float* beta, const float* alpha, const float* S0, const void* g,
                                     const float* w, void* y, float* ST, void* h_clvr, const float* clvr_scale,
                                     void* ws, size_t ws_bytes, void* stream) {
    if (desc && desc->B * desc->T * desc->H > 0 && !g) return fail(GDR_ERR_INVALID_ARG, "g is required");
    return forward_impl(desc, q, k, v, beta, alpha, S0, y, ST, h_clvr, clvr_scale, ws, ws_bytes, stream, false, g,
                        w);
}

gdr_status gdr_forward_train(const gdr_desc* desc, const void* q, const void* k, const void* v,
                             const float* beta, const float* alpha, const float* S0, void* o, float* ST,
                             void* h_clvr, const float* clvr_scale, void* ws, size_t ws_bytes,
                             void* stream) {
    return forward_impl(desc, q, k, v, beta, alpha, S0, o, ST, h_clvr, clvr_scale, ws, ws_bytes, stream, true);
}

gdr_status gdr_backward(const gdr_desc* desc, const void* q, const void* k, const void* v,
                        const float* beta, const float* alpha, const float* S0, const void* dO,
                        const float* dST, const void* dh_clvr, const float* clvr_scale, void* dq,
                        void* dk, void* dv, float* dbeta, float* dalpha, float* dS0,
                        float* dclvr_scale, void* ws, size_t ws_bytes, void* stream) {
    return backward_impl(desc, q, k, v, beta, alpha, S0, dO, dST, dh_clvr, clvr_scale, dq, dk, dv, dbeta,
                         dalpha, dS0, dclvr_scale, ws, ws_bytes, stream, true);
}

gdr_status gdr_backward_saved(const gdr_desc* desc, const void* q, const void* k, const void* v,
                              const float* beta, const float* alpha, const float* S0, const void* dO,
                              const float* dST, const void* dh_clvr, const float* clvr_scale, void* dq,
                              void* dk, void* dv, float* dbeta, float* dalpha, float* dS0,
                              float* dclvr_scale, void* ws, size_t ws_bytes, void* stream) {
    return backward_impl(desc, q, k, v, beta, alpha, S0, dO, dST, dh_clvr, clvr_scale, dq, dk, dv, dbeta,
                         dalpha, dS0, dclvr_scale, ws, ws_bytes, stream, false);
}

gdr_status gdr_decode_step(int64_t N, int64_t H, int64_t dk, int64_t dv, int32_t gate,
                           int32_t in_dtype, int32_t out_dtype, float scale, const void* q,
                           const void* k, const void* v, const float* beta, const float* alpha,
                           float* S, void* o, void* stream) {
    gdr_desc d;
    std::memset(&d, 0, sizeof d);
    d.B = N; d.T = 1; d.H = H; d.dk = dk; d.dv = dv; d.gate = gate; d.in_dtype = in_dtype;
    d.out_dtype = out_dtype; d.scale = scale; d.chunk = 0;
    gdr_status st = check_desc(&d, nullptr);
    if (st != GDR_OK) return st;
    const int64_t nslab = N * H;
    if (nslab == 0) return GDR_OK;
    if (nslab > 2147483647LL) return fail(GDR_ERR_INVALID_ARG, "N*H too large for one launch");
    if (!q || !k || !v || !beta || !S || !o)
        return fail(GDR_ERR_INVALID_ARG, "q, k, v, beta, S and o are required");
    if ((gate == GDR_GATE_NONE) != (alpha == nullptr))
        return fail(GDR_ERR_INVALID_ARG, "alpha must be NULL iff the gate is NONE");
    const void* ptrs[] = {q, k, v, beta, alpha, S, o};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(GDR_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
    const size_t ib = dtype_bytes(in_dtype), ob = dtype_bytes(out_dtype);
    const size_t n = size_t(nslab) * dk;
    const size_t s_bytes = size_t(nslab) * dk * dv * 4;
    const size_t a_bytes = gate == GDR_GATE_CHANNEL ? n * 4 : size_t(nslab) * 4;
    struct {
        const void* p;
        size_t n;
    } ins[] = {{q, n * ib}, {k, n * ib}, {v, n * ib}, {beta, size_t(nslab) * 4}, {alpha, a_bytes}};
    for (auto& in : ins) {
        if (overlap(o, n * ob, in.p, in.n)) return fail(GDR_ERR_INVALID_ARG, "o overlaps an input");
        if (overlap(S, s_bytes, in.p, in.n)) return fail(GDR_ERR_INVALID_ARG, "S overlaps an input");
    }
    if (overlap(S, s_bytes, o, n * ob)) return fail(GDR_ERR_INVALID_ARG, "o overlaps S");
    hipStream_t s = static_cast<hipStream_t>(stream);
    {
        const bool bf = in_dtype != GDR_FP32;
        const uint32_t F = gdr::CHECK_FINITE;
        const Check checks[] = {
            {q, int64_t(n), bf, F, "q"}, {k, int64_t(n), bf, F, "k"}, {v, int64_t(n), bf, F, "v"},
            {beta, nslab, false, F, "beta"}, {alpha, int64_t(a_bytes / 4), false, gdr::CHECK_ALPHA_CLOSED, "alpha"},
            {S, int64_t(s_bytes / 4), false, F, "S"},
        };
        gdr_status g = run_checks(checks, int(sizeof checks / sizeof checks[0]), s);
        if (g != GDR_OK) return g;
    }
    gdr::prof_before(s);
    hipError_t e = gdr::launch_decode(int(dk), gate, in_dtype == GDR_FP32, out_dtype == GDR_FP32, nslab,
                                      int(H), scale, q, k, v, beta, alpha, S, o, s);
    gdr::prof_after("decode", s);
    if (e != hipSuccess) return fail(GDR_ERR_DEVICE, "decode launch: %s", hipGetErrorString(e));
    return GDR_OK;
}

// Output gate: one row of dv channels per token and head
static gdr_status gate_common(const gdr_desc* desc, int64_t* BT) {
    gdr_status st = check_desc(desc, nullptr);
    if (st != GDR_OK) return st;
    *BT = desc->B * desc->T;
    if (*BT * desc->H > 2147483647LL * 64) return fail(GDR_ERR_INVALID_ARG, "tensor too large");
    return GDR_OK;
}

gdr_status gdr_output_gate_forward(const gdr_desc* desc, const void* o, const void* g, const float* w, void* y,
                                   void* stream) {
    int64_t BT = 0;
    gdr_status st = gate_common(desc, &BT);
    if (st != GDR_OK) return st;
    const int64_t H = desc->H, D = desc->dv;
    if (BT * H == 0) return GDR_OK;
    if (!o || !g || !y) return fail(GDR_ERR_INVALID_ARG, "o, g and y are required");
    const void* ptrs[] = {o, g, w, y};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(GDR_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
    const size_t n = size_t(BT) * H * D;
    const size_t ob = dtype_bytes(desc->out_dtype), ib = dtype_bytes(desc->in_dtype);
    if (overlap(y, n * ob, g, n * ib) || overlap(y, n * ob, w, size_t(H) * D * 4))
        return fail(GDR_ERR_INVALID_ARG, "y overlaps g or w");
    if (y != o && overlap(y, n * ob, o, n * ob))
        return fail(GDR_ERR_INVALID_ARG, "y partially overlaps o (it may only be o itself)");
    hipStream_t s = static_cast<hipStream_t>(stream);
    {
        const uint32_t F = gdr::CHECK_FINITE;
        const Check checks[] = {{o, int64_t(n), desc->out_dtype != GDR_FP32, F, "o"},
                                {g, int64_t(n), desc->in_dtype != GDR_FP32, F, "g"},
                                {w, H * D, false, F, "w"}};
        gdr_status gs = run_checks(checks, 3, s);
        if (gs != GDR_OK) return gs;
    }
    gdr::prof_before(s);
    hipError_t e = gdr::launch_gate(false, int(D), desc->in_dtype == GDR_FP32, desc->out_dtype == GDR_FP32, BT, int(H),
                                    o, g, w, y, nullptr, nullptr, nullptr, nullptr, nullptr, s);
    gdr::prof_after("gate_fwd", s);
    if (e != hipSuccess) return fail(GDR_ERR_DEVICE, "output-gate launch: %s", hipGetErrorString(e));
    return GDR_OK;
}

size_t gdr_output_gate_workspace_size(const gdr_desc* desc) {
    int64_t BT = 0;
    if (gate_common(desc, &BT) != GDR_OK) return 0;
    return align_up(size_t(gdr::gate_segments(BT)) * size_t(desc->H) * size_t(desc->dv) * 4);
}

gdr_status gdr_output_gate_backward(const gdr_desc* desc, const void* o, const void* g, const float* w,
                                    const void* dy, void* dO, void* dg, float* dw, void* ws, size_t ws_bytes,
                                    void* stream) {
    int64_t BT = 0;
    gdr_status st = gate_common(desc, &BT);
    if (st != GDR_OK) return st;
    const int64_t H = desc->H, D = desc->dv;
    if (BT * H == 0) return GDR_OK;
    if (!o || !g || !dy || !dO || !dg) return fail(GDR_ERR_INVALID_ARG, "o, g, dy, dO and dg are required");
    const void* ptrs[] = {o, g, w, dy, dO, dg, dw, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(GDR_ERR_INVALID_ARG, "pointer %p is not 16-byte aligned", p);
    const size_t n = size_t(BT) * H * D;
    const size_t ob = dtype_bytes(desc->out_dtype), ib = dtype_bytes(desc->in_dtype);
    const size_t need = dw ? gdr_output_gate_workspace_size(desc) : 0;
    if (dw && (ws_bytes < need || !ws))
        return fail(GDR_ERR_WORKSPACE, "workspace too small: need %zu bytes, got %zu", need, ws_bytes);
    struct {
        const void* p;
        size_t n;
    } ins[] = {{o, n * ob}, {g, n * ib}, {w, size_t(H) * D * 4}, {dy, n * ob}},
      outs[] = {{dO, n * ib}, {dg, n * ib}, {dw, size_t(H) * D * 4}, {dw ? ws : nullptr, need}};
    for (auto& o1 : outs) {
        for (auto& in : ins)
            if (overlap(o1.p, o1.n, in.p, in.n)) return fail(GDR_ERR_INVALID_ARG, "an output overlaps an input");
        for (auto& o2 : outs)
            if (&o1 != &o2 && overlap(o1.p, o1.n, o2.p, o2.n)) return fail(GDR_ERR_INVALID_ARG, "two outputs overlap");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    {
        const uint32_t F = gdr::CHECK_FINITE;
        const Check checks[] = {{o, int64_t(n), desc->out_dtype != GDR_FP32, F, "o"},
                                {g, int64_t(n), desc->in_dtype != GDR_FP32, F, "g"},
                                {w, H * D, false, F, "w"},
                                {dy, int64_t(n), desc->out_dtype != GDR_FP32, F, "dy"}};
        gdr_status gs = run_checks(checks, 4, s);
        if (gs != GDR_OK) return gs;
    }
    gdr::prof_before(s);
    hipError_t e = gdr::launch_gate(true, int(D), desc->in_dtype == GDR_FP32, desc->out_dtype == GDR_FP32, BT, int(H),
                                    o, g, w, nullptr, dy, dO, dg, dw, static_cast<float*>(ws), s);
    gdr::prof_after("gate_bwd", s);
    if (e != hipSuccess) return fail(GDR_ERR_DEVICE, "output-gate launch: %s", hipGetErrorString(e));
    return GDR_OK;
}

}  // extern "C"
