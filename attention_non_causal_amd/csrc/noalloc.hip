// noalloc.hip -- dit_attn_fwd_noalloc: the split forward launch of
// dit_attn_fwd_ws with its scratch in a static device array instead of a
// caller-provided workspace, for callers that cannot allocate device memory
// (code under graph capture, tight serving loops, harnesses that forbid
// allocation).
//
// `scratch` is a file-scope device array: each GPU the library runs on holds
// its own copy (for as long as the process lives) at its own address.  In host
// code the array's name is only a host-side stand-in, never a device address,
// so the device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept; only that pointer
// is ever handed to kernels.  Every call on one GPU shares that GPU's array and
// leaves its last contents behind: nothing in it has to start at zero (each
// piece of a split tile writes all of its partial result before the merge
// kernel, later on the same stream, reads it).  Calls that overlap on one GPU
// (other streams, other host threads) race on the array.
#include "dit_attn.h"

#include <mutex>

#include "launch.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[DIT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (null: not looked up)

// Device address of the current device's scratch array, or nullptr.
void* scratch_on_current_device(int* status)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *status = DIT_ERR_HIP;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            *status = DIT_ERR_HIP;
            return nullptr;
        }
        g_scratch[dev] = p;
    }
    *status = DIT_OK;
    return g_scratch[dev];
}

}  // namespace

extern "C" int dit_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int B, int H, int Sq, int Skv, int d,
                                    float scale, int dtype, hipStream_t stream)
{
    // every argument is validated first; the scratch address is looked up only
    // for a launch that is split, and a shape whose split needs more than
    // DIT_NOALLOC_SCRATCH_BYTES returns DIT_ERR_WORKSPACE before that
    return dit::fwd_entry(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype, true, nullptr,
                          DIT_NOALLOC_SCRATCH_BYTES, false, 0, stream,
                          scratch_on_current_device);
}
