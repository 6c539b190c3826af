// Static device scratch of muon_step_noalloc: the entry point for callers that
// cannot allocate device memory.  Every buffer a step needs beyond the
// caller's tensors (workspace, tile lists, units, norm partials, descriptor
// table) lives in one file-scope array per GPU, reserved when the library's
// code object is loaded and held until the process ends.  In host code the
// array's name stands for a host-side symbol, not a device address, so its
// address on each device is looked up once with hipGetSymbolAddress (with that
// device current) and only that address is used afterwards.

#include <hip/hip_runtime.h>

#include <mutex>

#include "muon_internal.hpp"

namespace muon {
namespace {

static __device__ __align__(256) char scratch[kStaticScratchBytes];

struct ScratchAddr {
    std::once_flag once;
    hipError_t status = hipSuccess;
    char* ptr = nullptr;
};
ScratchAddr g_addr[kMaxStaticDevices];

}  // namespace

hipError_t static_scratch_base(int device, char** base) {
    if (device < 0 || device >= kMaxStaticDevices) return hipErrorInvalidDevice;
    ScratchAddr& a = g_addr[device];
    std::call_once(a.once, [&]() {
        void* p = nullptr;
        a.status = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (a.status == hipSuccess) a.ptr = static_cast<char*>(p);
        else (void)hipGetLastError();
    });
    *base = a.ptr;
    return a.status;
}

}  // namespace muon
