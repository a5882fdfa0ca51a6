// The library's own device scratch, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid it): the workspace of gdn_chunk_gated_delta_rule_fwd_noalloc.
//
// A file-scope device array of a fixed size, which every GPU the library runs
// on holds from when this code object is loaded on it until the process ends.
// In host code the name `scratch` stands for a host-side shadow, not the
// device array, so it is never passed anywhere: its address on a device is
// looked up once per device, with that device current, and only that address
// is used from then on.  Nothing in it needs clearing between calls (every
// value a kernel computes with was written by an earlier kernel of the same
// call; bytes staged but unused, such as the lo parts of P with bf16
// activations, may hold anything), but every call on one GPU uses the same
// bytes, so calls that may overlap on a GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

size_t scratch_bytes() { return kScratchBytes; }

hipError_t scratch_address(int device, void** out) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        int current = -1;
        hipError_t e = hipGetDevice(&current);
        if (e != hipSuccess) return e;
        if (current != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (current != device) {
            const hipError_t r = hipSetDevice(current);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = p;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

}  // namespace gdn
