// noalloc.hip -- the GQA shard decode partial without a caller workspace: its
// split-context partials live in a fixed device array of the library, so the
// call allocates nothing (for callers that cannot allocate device memory).
//
// The array is a file-scope __device__ variable: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  That
// address is looked up once per device (hipGetSymbolAddress, with the device
// current) on the device's first call and kept; the array's name itself is a
// host-side stand-in and is never passed to a kernel.
#include <mutex>

#include "internal.hpp"

namespace cpattn {
namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB per device
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// This device's copy of `scratch` (nullptr and an error message on failure).
void *device_scratch(cp_status *st) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *st = fail(CP_E_HIP, "gqa decode (no alloc): no current device (%s)",
                   hipGetErrorString(e));
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            *st = fail(CP_E_HIP, "gqa decode (no alloc): scratch address on device %d: %s", dev,
                       hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *st = CP_OK;
    return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace cpattn

using namespace cpattn;

extern "C" size_t cp_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" cp_status cp_decode_attn_partial_gqa_noalloc(const cp_gqa_args *a, hipStream_t stream) {
    clear_error();
    if (!a) return fail(CP_E_INVALID, "cp_decode_attn_partial_gqa_noalloc: NULL args");
    cp_status st = validate_gqa(a);  // the plan below assumes valid sizes
    if (st != CP_OK || a->B == 0) return st;
    const GqaPlan pl = plan_gqa(*a);
    if (pl.ws_bytes > kScratchBytes)
        return fail(CP_E_WORKSPACE,
                    "gqa decode (no alloc): %zu bytes of split partials needed, the built-in "
                    "scratch holds %zu",
                    pl.ws_bytes, kScratchBytes);
    void *ws = pl.ws_bytes > 0 ? device_scratch(&st) : nullptr;
    if (st != CP_OK) return st;
    return cp_decode_attn_partial_gqa(a, ws, ws ? kScratchBytes : 0, stream);
}
