// gdr_noalloc.hip -- gdr_forward_chunked_noalloc: the chunked forward with its
// workspace in a fixed device array of the library instead of a caller buffer.
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid it).  The array is a file-scope
// device symbol; each GPU the library runs on holds its own copy for the life
// of the process.  Its device address is taken once per device, with that
// device current, by hipGetSymbolAddress; the host-side name of the array is
// never passed to a kernel or a copy.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdio>
#include <mutex>

#include "../../include/gdr.h"

namespace gdr {
// The forward of gdr_abi.cpp (argument checks, workspace carving, launches).
gdr_status forward_entry(const gdr_desc* desc, const void* q, const void* k, const void* v, const float* beta,
                         const float* alpha, const float* S0, void* o, float* ST, void* h_clvr,
                         const float* clvr_scale, void* ws, size_t ws_bytes, void* stream);
gdr_status set_error(gdr_status s, const char* msg);
}  // namespace gdr

static constexpr size_t kScratchBytes = size_t(GDR_NOALLOC_SCRATCH_BYTES);

// The workspace of gdr_forward_chunked_noalloc on every GPU.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch`, or nullptr (the error is set).
void* device_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        gdr::set_error(GDR_ERR_DEVICE, "no current device");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            gdr::set_error(GDR_ERR_DEVICE, "the library's scratch array has no device address");
            return nullptr;
        }
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" {

size_t gdr_noalloc_scratch_bytes(void) { return kScratchBytes; }

gdr_status gdr_forward_chunked_noalloc(const gdr_desc* desc, const void* q, const void* k, const void* v,
                                       const float* beta, const float* alpha, const float* S0, void* o,
                                       float* ST, void* h_clvr, const float* clvr_scale, void* stream) {
    const size_t need = gdr_workspace_size(desc, 0);
    if (need == 0 && desc && desc->B * desc->T * desc->H > 0)
        return GDR_ERR_INVALID_ARG;  // gdr_workspace_size has set the reason
    if (need > kScratchBytes) {
        char msg[192];
        std::snprintf(msg, sizeof msg,
                      "the forward needs %zu bytes of workspace, above the %zu-byte scratch array of the "
                      "allocation-free entry point; call gdr_forward_chunked with a workspace instead",
                      need, kScratchBytes);
        return gdr::set_error(GDR_ERR_WORKSPACE, msg);
    }
    void* ws = need ? device_scratch() : nullptr;
    if (need && !ws) return GDR_ERR_DEVICE;
    return gdr::forward_entry(desc, q, k, v, beta, alpha, S0, o, ST, h_clvr, clvr_scale, ws, kScratchBytes,
                              stream);
}

}  // extern "C"
