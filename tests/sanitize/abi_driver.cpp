// Drives the host side of the C ABI (include/gdr.h) under the address and
// undefined-behaviour sanitizers, with the kernel launchers replaced by the
// stand-ins of abi_stubs.cpp.  The ABI never dereferences a tensor pointer on
// the host, so ordinary host buffers stand in for device memory.  Exits
// non-zero (or the sanitizers abort) on the first failure.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/gdr.h"

namespace stub {
extern const char* ws_lo;
extern const char* ws_hi;
extern long launches;
}  // namespace stub

static int g_fail = 0;
#define EXPECT(cond, ...)                                                   \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);       \
            std::fprintf(stderr, __VA_ARGS__);                              \
            std::fprintf(stderr, " (last error: %s)\n", gdr_last_error()); \
            ++g_fail;                                                       \
        }                                                                   \
    } while (0)

// 256-byte aligned host block standing in for one device tensor
struct Buf {
    std::vector<char> mem;
    char* p;
    explicit Buf(size_t n) : mem(n + 512), p(mem.data() + (256 - reinterpret_cast<uintptr_t>(mem.data()) % 256)) {}
};

static gdr_desc desc(int64_t B, int64_t T, int64_t H, int64_t d, int gate, int in, int out, int route = 0,
                     int pro = 0) {
    gdr_desc x;
    std::memset(&x, 0, sizeof x);
    x.B = B; x.T = T; x.H = H; x.dk = d; x.dv = d; x.gate = gate; x.in_dtype = in; x.out_dtype = out;
    x.scale = 1.0f; x.chunk = 0; x.route = route; x.prologue = pro;
    return x;
}

// One forward and one backward with every optional tensor given, through the
// launch stand-ins; returns the statuses.
static void run_pair(const gdr_desc& d, bool train) {
    const size_t ib = d.in_dtype == GDR_FP32 ? 4 : 2, ob = d.out_dtype == GDR_FP32 ? 4 : 2;
    const size_t n = size_t(d.B * d.T * d.H * d.dk), nt = size_t(d.B * d.T * d.H);
    const size_t na = d.gate == GDR_GATE_CHANNEL ? n : nt;
    const size_t ns = size_t(d.B * d.H * d.dk * d.dv);
    Buf q(n * ib), k(n * ib), v(n * ib), beta(nt * 4), alpha(na * 4), S0(ns * 4), o(n * ob), ST(ns * 4),
        h(n * ib), lam(size_t(d.H * d.dv) * 4), dO(n * ib), dST(ns * 4), dh(n * ib), dq(n * ob), dk(n * ob),
        dv(n * ob), dbeta(nt * 4), dalpha(na * 4), dS0(ns * 4), dlam(size_t(d.H * d.dv) * 4);
    const float* al = d.gate == GDR_GATE_NONE ? nullptr : reinterpret_cast<float*>(alpha.p);
    float* dal = d.gate == GDR_GATE_NONE ? nullptr : reinterpret_cast<float*>(dalpha.p);
    const size_t wf = gdr_workspace_size(&d, train ? 1 : 0), wb = gdr_workspace_size(&d, 1);
    EXPECT(wf > 0 || n == 0, "workspace size 0 for a valid descriptor");
    Buf ws(wb > wf ? wb : wf);
    stub::ws_lo = ws.p;
    stub::ws_hi = ws.p + (wb > wf ? wb : wf);
    auto F = [](char* p) { return reinterpret_cast<float*>(p); };
    gdr_status s = (train ? gdr_forward_train : gdr_forward_chunked)(
        &d, q.p, k.p, v.p, F(beta.p), al, F(S0.p), o.p, F(ST.p), h.p, F(lam.p), ws.p, wf, nullptr);
    EXPECT(s == GDR_OK, "forward status %d", int(s));
    s = (train ? gdr_backward_saved : gdr_backward)(&d, q.p, k.p, v.p, F(beta.p), al, F(S0.p), dO.p, F(dST.p),
                                                    dh.p, F(lam.p), dq.p, dk.p, dv.p, F(dbeta.p), dal, F(dS0.p),
                                                    F(dlam.p), ws.p, wb, nullptr);
    EXPECT(s == GDR_OK, "backward status %d", int(s));
    // a workspace one byte short is refused before anything runs
    const long before = stub::launches;
    if (wf > 0) {
        s = gdr_forward_chunked(&d, q.p, k.p, v.p, F(beta.p), al, F(S0.p), o.p, F(ST.p), nullptr, nullptr, ws.p,
                                gdr_workspace_size(&d, 0) - 1, nullptr);
        EXPECT(s == GDR_ERR_WORKSPACE, "short workspace status %d", int(s));
    }
    // an output overlapping an input is refused
    if (n > 0) {
        s = gdr_forward_chunked(&d, q.p, k.p, v.p, F(beta.p), al, F(S0.p), q.p, nullptr, nullptr, nullptr, ws.p,
                                wf, nullptr);
        EXPECT(s == GDR_ERR_INVALID_ARG, "o aliasing q: status %d", int(s));
        s = gdr_forward_chunked(&d, q.p + 2, k.p, v.p, F(beta.p), al, F(S0.p), o.p, nullptr, nullptr, nullptr,
                                ws.p, wf, nullptr);
        EXPECT(s == GDR_ERR_INVALID_ARG, "misaligned q: status %d", int(s));
    }
    EXPECT(stub::launches == before, "a refused call launched");
    stub::ws_lo = stub::ws_hi = nullptr;
}

int main() {
    // descriptor checks and workspace sizes over a grid of shapes
    const int64_t Ts[] = {0, 1, 63, 64, 65, 130, 1000, 5000};
    for (int64_t T : Ts)
        for (int d : {64, 128})
            for (int gate = 0; gate < 3; ++gate)
                for (int in = 0; in < 2; ++in)
                    for (int route = 0; route < 2; ++route)
                        for (int pro = 0; pro < 3; ++pro) {
                            gdr_desc x = desc(2, T, 3, d, gate, in, in, route, pro);
                            const size_t f = gdr_workspace_size(&x, 0), b = gdr_workspace_size(&x, 1);
                            EXPECT(T == 0 || (f > 0 && b > f), "sizes %zu %zu", f, b);
                        }
    gdr_desc bad = desc(1, 64, 1, 96, 2, 0, 0);
    EXPECT(gdr_workspace_size(&bad, 0) == 0, "d = 96 accepted");
    bad = desc(1, 64, 1, 64, 7, 0, 0);
    EXPECT(gdr_workspace_size(&bad, 0) == 0, "gate 7 accepted");
    bad = desc(-1, 64, 1, 64, 2, 0, 0);
    EXPECT(gdr_workspace_size(&bad, 0) == 0, "B = -1 accepted");
    bad = desc(1, 64, 1, 64, 2, 0, 0);
    bad.chunk = 32;
    EXPECT(gdr_workspace_size(&bad, 0) == 0, "chunk 32 accepted");
    EXPECT(gdr_workspace_size(nullptr, 0) == 0, "NULL descriptor accepted");
    bad = desc(int64_t(1) << 41, 64, 1, 64, 2, 0, 0);
    EXPECT(gdr_workspace_size(&bad, 0) == 0, "huge B accepted");

    // full argument paths through the launch stand-ins
    for (int train = 0; train < 2; ++train)
        for (int gate = 0; gate < 3; ++gate)
            for (int in = 0; in < 2; ++in)
                for (int route = 0; route < 2; ++route)
                    for (int pro = 0; pro < 3; pro += 2)
                        for (int64_t T : {int64_t(1), int64_t(65), int64_t(300)}) {
                            const int d = in == GDR_FP32 ? 64 : 128;
                            run_pair(desc(2, T, 2, d, gate, in, GDR_FP32, route, pro), train != 0);
                        }
    // fp32 at d = 128: the two-kernel gradient path, every route, with and without
    // the prologue
    for (int train = 0; train < 2; ++train)
        for (int route = 0; route < 2; ++route)
            for (int pro = 0; pro < 3; pro += 2)
                run_pair(desc(1, 200, 2, 128, 2, GDR_FP32, GDR_FP32, route, pro), train != 0);

    // the separate-gate variant (Gated DeltaNet-2): forward and decode
    for (int gate = 0; gate < 3; ++gate)
        for (int in = 0; in < 2; ++in)
            for (int64_t T : {int64_t(0), int64_t(1), int64_t(130)}) {
                const int64_t d = in == GDR_FP32 ? 64 : 128;
                gdr_desc x = desc(2, T, 3, d, gate, in, GDR_FP32);
                const size_t n = size_t(2 * T * 3 * d), ns = size_t(2 * 3 * d * d), ib = in == GDR_FP32 ? 4 : 2;
                const size_t na = gate == GDR_GATE_CHANNEL ? n : size_t(2 * T * 3);
                Buf q(n * ib), k(n * ib), v(n * ib), e(n * 4), w(n * 4), a(na * 4), S0(ns * 4), o(n * 4), ST(ns * 4);
                const size_t need = gdr_gdn2_workspace_size(&x);
                EXPECT(T == 0 || need > 0, "gdn2 workspace size 0");
                Buf ws(need);
                stub::ws_lo = ws.p;
                stub::ws_hi = ws.p + need;
                auto F = [](char* p) { return reinterpret_cast<float*>(p); };
                const float* al = gate == GDR_GATE_NONE ? nullptr : F(a.p);
                EXPECT(gdr_gdn2_forward_chunked(&x, q.p, k.p, v.p, F(e.p), F(w.p), al, F(S0.p), o.p, F(ST.p), ws.p,
                                                need, nullptr) == GDR_OK, "gdn2 forward");
                if (need > 0)
                    EXPECT(gdr_gdn2_forward_chunked(&x, q.p, k.p, v.p, F(e.p), F(w.p), al, F(S0.p), o.p, F(ST.p),
                                                    ws.p, need - 1, nullptr) == GDR_ERR_WORKSPACE,
                           "gdn2 short workspace");
                if (T > 0)
                    EXPECT(gdr_gdn2_forward_chunked(&x, q.p, k.p, v.p, F(e.p), F(w.p), al, F(S0.p), e.p, F(ST.p),
                                                    ws.p, need, nullptr) == GDR_ERR_INVALID_ARG,
                           "gdn2 o aliasing erase");
                gdr_desc xr = x;
                xr.route = GDR_ROUTE_ERROR;
                EXPECT(gdr_gdn2_workspace_size(&xr) == 0, "gdn2 with a route accepted");
                stub::ws_lo = stub::ws_hi = nullptr;
                if (T == 1)
                    EXPECT(gdr_gdn2_decode_step(2, 3, d, d, gate, in, GDR_FP32, 1.f, q.p, k.p, v.p, F(e.p), F(w.p), al,
                                                F(S0.p), o.p, nullptr) == GDR_OK, "gdn2 decode");
            }

    // decode and the output gate
    {
        const int64_t N = 3, H = 2, d = 64;
        Buf q(N * H * d * 2), k(N * H * d * 2), v(N * H * d * 2), beta(N * H * 4), alpha(N * H * d * 4),
            S(N * H * d * d * 4), o(N * H * d * 4);
        auto F = [](char* p) { return reinterpret_cast<float*>(p); };
        EXPECT(gdr_decode_step(N, H, d, d, 2, 0, 1, 1.f, q.p, k.p, v.p, F(beta.p), F(alpha.p), F(S.p), o.p,
                               nullptr) == GDR_OK, "decode");
        EXPECT(gdr_decode_step(N, H, d, d, 2, 0, 1, 1.f, q.p, k.p, v.p, F(beta.p), nullptr, F(S.p), o.p,
                               nullptr) == GDR_ERR_INVALID_ARG, "decode without alpha");
        EXPECT(gdr_decode_step(N, H, d, d, 2, 0, 1, 1.f, q.p, k.p, v.p, F(beta.p), F(alpha.p), F(S.p), S.p,
                               nullptr) == GDR_ERR_INVALID_ARG, "decode o aliasing S");
        gdr_desc x = desc(2, 100, 2, 64, 0, 0, 0);
        Buf oo(2 * 100 * 2 * 64 * 2), g(2 * 100 * 2 * 64 * 2), w(2 * 64 * 4), y(2 * 100 * 2 * 64 * 2),
            dy(2 * 100 * 2 * 64 * 2), dO(2 * 100 * 2 * 64 * 2), dg(2 * 100 * 2 * 64 * 2), dw(2 * 64 * 4);
        Buf gws(gdr_output_gate_workspace_size(&x));
        stub::ws_lo = gws.p;
        stub::ws_hi = gws.p + gdr_output_gate_workspace_size(&x);
        EXPECT(gdr_output_gate_forward(&x, oo.p, g.p, F(w.p), y.p, nullptr) == GDR_OK, "gate forward");
        EXPECT(gdr_output_gate_forward(&x, oo.p, g.p, F(w.p), oo.p, nullptr) == GDR_OK, "gate in place");
        EXPECT(gdr_output_gate_backward(&x, oo.p, g.p, F(w.p), dy.p, dO.p, dg.p, F(dw.p), gws.p,
                                        gdr_output_gate_workspace_size(&x), nullptr) == GDR_OK, "gate backward");
        EXPECT(gdr_output_gate_backward(&x, oo.p, g.p, F(w.p), dy.p, dO.p, dg.p, F(dw.p), gws.p, 4, nullptr) ==
                   GDR_ERR_WORKSPACE, "gate backward short workspace");
        stub::ws_lo = stub::ws_hi = nullptr;
    }

    // the debug mode asks the device: without one, a valid call reports a device error
    setenv("GDR_VALIDATE", "1", 1);
    {
        gdr_desc x = desc(1, 70, 1, 64, 2, 0, 1);
        const size_t n = 70 * 64;
        Buf q(n * 2), k(n * 2), v(n * 2), beta(70 * 4), alpha(n * 4), o(n * 4);
        Buf ws(gdr_workspace_size(&x, 0));
        auto F = [](char* p) { return reinterpret_cast<float*>(p); };
        const long before = stub::launches;
        const gdr_status s = gdr_forward_chunked(&x, q.p, k.p, v.p, F(beta.p), F(alpha.p), nullptr, o.p, nullptr,
                                                 nullptr, nullptr, ws.p, gdr_workspace_size(&x, 0), nullptr);
        EXPECT(s == GDR_ERR_DEVICE, "validate without a device: status %d", int(s));
        EXPECT(stub::launches == before, "validate without a device launched");
    }
    unsetenv("GDR_VALIDATE");

    EXPECT(std::strcmp(gdr_status_string(GDR_ERR_WORKSPACE), "GDR_ERR_WORKSPACE") == 0, "status string");
    std::printf("abi driver: %ld stand-in launches, %d failures\n", stub::launches, g_fail);
    return g_fail ? 1 : 0;
}
