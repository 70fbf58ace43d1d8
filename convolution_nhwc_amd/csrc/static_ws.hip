// cnhwc_fwd_static_ws: the forward pass with its workspace in a device array
// of the library instead of a caller-allocated buffer, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ variable: the code object reserves it
// on every GPU the library's kernels are loaded on, and it stays reserved
// until the process ends.  Its device address differs per GPU and is not the
// host-side name of the array, so it is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.  The forward kernels that use a workspace overwrite
// every byte they later read (split-C partial sums, the implicit-GEMM
// forward's transformed filter), so nothing in it has to start at zero.
#include <mutex>
#include <string>

#include "internal.h"

namespace cnhwc {
namespace {

constexpr size_t kStaticWsBytes = CNHWC_STATIC_WS_BYTES;   // 32 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticWsBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on first use).
int scratch_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return set_error(CNHWC_HIP_ERROR, std::string("hipGetDevice failed: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return set_error(CNHWC_HIP_ERROR, "device index " + std::to_string(dev) + " out of range");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return set_error(CNHWC_HIP_ERROR, std::string("hipGetSymbolAddress of the static workspace failed: ") +
                                                  hipGetErrorString(e));
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return CNHWC_OK;
}

}  // namespace
}  // namespace cnhwc

extern "C" int cnhwc_fwd_static_ws(const cnhwc_problem* prob, const void* x, const void* w, void* y,
                                   void* hip_stream) {
    using namespace cnhwc;
    size_t need = 0;
    int st = cnhwc_workspace_size(prob, CNHWC_OP_FWD, &need);
    if (st) return st;
    if (need > kStaticWsBytes)
        return set_error(CNHWC_WORKSPACE_TOO_SMALL,
                         "the forward kernel for this problem needs " + std::to_string(need) +
                             " workspace bytes; the static workspace holds " + std::to_string(kStaticWsBytes) +
                             " (use cnhwc_fwd with a caller-allocated workspace)");
    void* ws = nullptr;
    if (need > 0 && (st = scratch_ptr(&ws))) return st;
    return cnhwc_fwd(prob, x, w, y, ws, need > 0 ? kStaticWsBytes : 0, hip_stream);
}
