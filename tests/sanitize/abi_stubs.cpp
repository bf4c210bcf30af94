// Host-only stand-ins for the kernel launchers of libgdr, for building the C ABI
// layer (gdr_abi.cpp) with the address and undefined-behaviour sanitizers on a
// machine without a GPU.  Each stand-in checks that every workspace pointer the
// ABI layer carved lies inside the buffer the driver registered, counts the
// call and launches nothing.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "../../gated_delta_rule_37_amd/csrc/gdr_gate.hpp"
#include "../../gated_delta_rule_37_amd/csrc/gdr_launch.hpp"

namespace stub {
const char* ws_lo = nullptr;
const char* ws_hi = nullptr;
long launches = 0;
}  // namespace stub

namespace {

void in_ws(const void* p, const char* what) {
    // an empty workspace (no chunks) carves pointers that are never read
    if (!p || !stub::ws_lo || stub::ws_lo == stub::ws_hi) return;
    const char* c = static_cast<const char*>(p);
    if (c < stub::ws_lo || c >= stub::ws_hi) {
        std::fprintf(stderr, "workspace pointer %s outside the workspace\n", what);
        std::abort();
    }
}

void check_ws(const gdr::ChunkWs& w) {
    const void* ps[] = {w.W,  w.Ut,  w.Qt,     w.KbT,    w.A,       w.gam,  w.AT,  w.Kb,  w.QtT,
                        w.WT, w.Nw,  w.Pw,     w.Ssnap,  w.Usave,   w.dSsnap, w.dUsave, w.dUsaveT,
                        w.gQt, w.gKt, w.gKb,   w.gA,     w.gP,      w.gGam, w.Mt,  w.Bact, w.rq, w.rk};
    for (const void* p : ps) in_ws(p, "ChunkWs");
}

void check_range(gdr::ChunkRange cr, int64_t NC) {
    if (cr.lo < 0 || cr.n < 1 || cr.lo + cr.n > NC) {
        std::fprintf(stderr, "chunk range [%lld, +%lld) outside [0, %lld)\n", (long long)cr.lo, (long long)cr.n,
                     (long long)NC);
        std::abort();
    }
}

}  // namespace

namespace gdr {

hipError_t launch_decode(int, int, bool, bool, int64_t, int, float, const void*, const void*, const void*,
                         const float*, const float*, float*, void*, hipStream_t) {
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_output_gated(int, bool, int64_t, int64_t, int, int64_t NC, float, const ChunkWs& ws, void*,
                               const float*, const float*, void*, const OutGate& og, ChunkRange cr, hipStream_t) {
    if (!og.g) std::abort();
    check_ws(ws);
    check_range(cr, NC);
    ++stub::launches;
    return hipSuccess;
}

hipError_t launch_output(int, bool, int64_t, int64_t, int, int64_t NC, float, const ChunkWs& ws, void*,
                         const float*, const float*, void*, ChunkRange cr, hipStream_t) {
    check_ws(ws);
    check_range(cr, NC);
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_intra(int, int, bool, int, int64_t, int64_t, int, int64_t NC, const void*, const void*,
                        const void*, const float*, const float*, void*, const float*, const ChunkWs& ws, int,
                        ChunkRange cr, hipStream_t) {
    check_ws(ws);
    check_range(cr, NC);
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_state_fwd(int, bool, bool, int64_t, int64_t, int, int64_t NC, float, const ChunkWs& ws,
                            const float* S0, float* ST, void*, bool, bool, ChunkRange cr, hipStream_t) {
    check_ws(ws);
    if (NC > 0) check_range(cr, NC);
    (void)S0;
    (void)ST;
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_state_bwd(int, bool, int64_t, int64_t, int, int64_t NC, float, const ChunkWs& ws, const void*,
                            const float*, float*, const void*, const float*, const float*, bool, ChunkRange cr,
                            hipStream_t) {
    check_ws(ws);
    if (NC > 0) check_range(cr, NC);
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_grads(int, int, bool, bool, int64_t, int64_t, int, int64_t NC, float, const void*, const void*,
                        const void*, const float*, const float*, const void*, const void*, const float*, void*,
                        void*, void*, float*, float*, const ChunkWs& ws, int, ChunkRange cr, bool, float* partial,
                        int ahead, hipStream_t) {
    if (ahead < 0 || ahead % 8) {
        std::fprintf(stderr, "launch_grads: prefetch distance %d\n", ahead);
        std::abort();
    }
    check_ws(ws);
    check_range(cr, NC);
    in_ws(partial, "partial");
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_clvr_dlam(bool, int64_t, int, int, const void*, const void*, float*, float* partial, int64_t,
                            hipStream_t) {
    in_ws(partial, "partial");
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_dlam_final(int, int64_t, const float* partial, float*, hipStream_t) {
    in_ws(partial, "partial");
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_cler_fwd(int, bool, int64_t, int64_t, int, int64_t, const ChunkWs& ws, const float*,
                           const float*, void*, hipStream_t) {
    check_ws(ws);
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_cler_mt(int, bool, int64_t, int64_t, int, int64_t, const ChunkWs& ws, const float*, const void*,
                          hipStream_t) {
    check_ws(ws);
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_state_fwd_xy(int, bool, bool, int64_t, int64_t, int, int64_t NC, float, const ChunkWs& ws,
                               const float*, float*, void*, ChunkRange cr, hipStream_t) {
    if (NC > 0) check_range(cr, NC);
    check_ws(ws);
    in_ws(ws.X, "X");
    in_ws(ws.Y, "Y");
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_gdn2_intra(int, int, bool, int64_t, int64_t, int, int64_t NC, const void*, const void*,
                             const void*, const float*, const float*, const float*, const ChunkWs& ws, ChunkRange cr,
                             hipStream_t) {
    check_range(cr, NC);
    check_ws(ws);
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_gdn2_decode(int, int, bool, bool, int64_t, float, const void*, const void*, const void*,
                              const float*, const float*, const float*, float*, void*, hipStream_t) {
    ++stub::launches;
    return hipSuccess;
}
int64_t gate_segments(int64_t BT) { return BT < 1 ? 1 : (BT < 256 ? BT : 256); }
hipError_t launch_gate(bool, int, bool, bool, int64_t, int, const void*, const void*, const float*, void*,
                       const void*, void*, void*, float*, float* partial, hipStream_t) {
    in_ws(partial, "partial");
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_check(const void*, int64_t, bool, uint32_t, unsigned long long*, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t check_result_address(unsigned long long**) { return hipErrorNoDevice; }

}  // namespace gdr
