// Scratch memory of moe_decode_noalloc: a file-scope device array that the
// library owns, for callers that cannot allocate (code under HIP graph
// capture, serving loops, harnesses that forbid hipMalloc).
//
// Each GPU the library runs on holds its own copy of `scratch` at its own
// address, for the life of the process.  Host code never uses the array's
// name as a device address: on the first call on a device (with that device
// current) hipGetSymbolAddress resolves that device's copy, and the pointer
// is kept per device and passed to the kernels like any workspace.  Every
// call on one GPU shares that GPU's copy.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "ql_internal.h"

static __device__ __align__(256) unsigned char scratch[QL_DECODE_SCRATCH_BYTES];

namespace ql {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[kMaxDevices] = {};
std::atomic<bool> g_scratch_ready[kMaxDevices];
}  // namespace

int decode_scratch(unsigned char** ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QL_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return QL_ERR_UNSUPPORTED_SHAPE;
    if (!g_scratch_ready[dev].load(std::memory_order_acquire)) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_ready[dev].load(std::memory_order_relaxed)) {
            void* p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
                return QL_ERR_HIP;
            g_scratch_ptr[dev] = static_cast<unsigned char*>(p);
            g_scratch_ready[dev].store(true, std::memory_order_release);
        }
    }
    *ptr = g_scratch_ptr[dev];
    return QL_OK;
}

}  // namespace ql
