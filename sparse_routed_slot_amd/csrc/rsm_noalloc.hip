// rsm_noalloc.hip -- rsm_forward_chunked_noalloc: the chunked forward with its workspace in
// a fixed device array of the library instead of a caller buffer, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops).
//
// The array (`scratch`, kScratchBytes) lives in the code object: each device the library
// runs on holds its own copy until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol); the device address
// is looked up once per device with hipGetSymbolAddress, with that device current, and
// kept.  Every call on a device uses that device's one array, so calls that overlap on one
// device (different streams, or several host threads) race; the forward needs no zeroed
// workspace, so nothing is cleared between calls.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/rsm.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of the current device's array (looked up on the first call on a device).
int scratch_ptr(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RSM_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RSM_ERR_HIP;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return RSM_OK;
}

}  // namespace

extern "C" {

size_t rsm_noalloc_scratch_bytes(void) { return kScratchBytes; }

int rsm_forward_chunked_noalloc(const void* q, const void* k, const void* z, const void* v, int dtype,
                                const float* f, const float* H0, int64_t B, int64_t T, int64_t Hh, int64_t M,
                                int64_t Dv, int64_t K, int64_t C, float* o, float* H_out, int32_t* idx_out,
                                void* stream) {
    // sizes first: an oversized problem is refused before any device call
    const size_t need = rsm_forward_workspace_bytes(dtype, B, T, Hh, M, Dv, C, K);
    if (need > kScratchBytes) return RSM_ERR_TOO_LARGE;
    void* ws = nullptr;
    if (need > 0) {
        const int st = scratch_ptr(&ws);
        if (st != RSM_OK) return st;
    }
    return rsm_forward_chunked(q, k, z, v, dtype, f, H0, B, T, Hh, M, Dv, K, C, o, H_out, idx_out, ws,
                               need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"
