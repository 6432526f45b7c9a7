// k_noalloc.hip -- dr_forward_noalloc: the kind-generic forward with its
// workspace taken from a fixed device array instead of the caller, for
// callers that cannot allocate device memory.
//
// The array `scratch` is a file-scope device variable of kScratchBytes.  The
// runtime places one copy on every GPU the library's code is loaded on, and
// each copy lives until the process ends.  In host code the name `scratch`
// is only a host-side stand-in for the symbol, never a device address: its
// device address is looked up with hipGetSymbolAddress, once per device with
// that device current, and only that address is handed to the kernels.
#include <mutex>

#include "host.h"

namespace {

constexpr size_t kScratchBytes = (size_t)DR_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

// The current device's copy of `scratch`, looked up on first use.
dr_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DR_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DR_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DR_OK;
}

}  // namespace

extern "C" {

size_t dr_noalloc_scratch_bytes(void) { return kScratchBytes; }

dr_status dr_forward_noalloc(int kind, const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const float* h0, void* o, float* hT, int B, int T, int H, int Dk,
                             int Dv, int C, int dtype, const dr_prologue* prologue, unsigned* flags, void* stream) {
    if (kind < 0 || kind > 2) return DR_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || T < 0) return DR_ERR_INVALID_ARG;
    const size_t need = dr_workspace_bytes(kind, B, T, H, Dk, Dv, C, dtype);
    if (need == 0 && T > 0) {
        // sizes the forward does not build; let it report which
        return drh::forward(kind, q, k, v, g, kind == DR_KIND_DECAY_LA ? nullptr : beta, h0, o, hT, B, T, H, Dk,
                            Dv, C, dtype, nullptr, 0, flags, stream, prologue);
    }
    if (need > kScratchBytes) return DR_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    const dr_status s = scratch_on_current_device(&ws);
    if (s != DR_OK) return s;
    // the forward writes every workspace byte it reads within the call, so
    // nothing left by an earlier call needs clearing
    return drh::forward(kind, q, k, v, g, kind == DR_KIND_DECAY_LA ? nullptr : beta, h0, o, hT, B, T, H, Dk, Dv, C,
                        dtype, ws, kScratchBytes, flags, stream, prologue);
}

}  // extern "C"
