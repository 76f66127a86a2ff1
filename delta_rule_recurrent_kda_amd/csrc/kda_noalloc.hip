// kda_noalloc.hip -- the library's fixed device buffer for the forward entry point that
// allocates nothing (kda_forward_noalloc).
//
// The buffer is a file-scope device array: every GPU the library runs on holds its own
// copy, at its own address, from the code object's load until the process ends. Host code
// never passes the array's name to a kernel (on the host that name is a stand-in, not a
// device address); it looks the address up once per device with hipGetSymbolAddress and
// passes that pointer. Calls on one device share the buffer and its last contents.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_internal.h"

namespace kda {
namespace {

// 32 MiB: the segment summaries of the fused scan (128 KB per segment and head) for up to
// 256 (segment, head) pairs, less the segment table of packs of more than 64 samples
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void** ptr)
{
    *ptr = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace kda
