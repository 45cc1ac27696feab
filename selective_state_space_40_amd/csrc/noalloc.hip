// ssm_scan_fwd_noalloc: the forward scan for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). A chunked plan needs scratch for the
// chunk summaries (the state entering each chunk, each chunk's end state
// from a zero start and its decay product); here it lives in one fixed
// file-scope device array instead of a caller workspace.
//
// Every GPU the library runs on holds its own copy of the array, at its own
// address, from the moment the library's code is loaded on it until the
// process ends. The host-side name of the array is only a stand-in for the
// symbol: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current, on the first call that
// needs it) and kept per device, and only that address is ever handed to a
// kernel. Every call on one GPU shares the array and the array keeps what
// the last call left in it. The chunked scan writes every scratch value it
// reads before reading it, so nothing needs clearing; calls that overlap on
// one GPU (other streams, other threads) race on the array.
#include <hip/hip_runtime.h>

#include <atomic>
#include <stddef.h>
#include <stdint.h>

#include "internal.h"
#include "mamba_scan.h"

namespace {

constexpr size_t kScratchBytes = MAMBA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size keeps 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];  // device address of `scratch`, per device

// The scratch of the current device for a plan that needs `bytes` of it.
int device_scratch(size_t bytes, void** ws) {
    if (bytes > kScratchBytes) return MAMBA_ERR_WORKSPACE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MAMBA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MAMBA_ERR_UNSUPPORTED;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // two threads may both get here first; they store the same address
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return MAMBA_ERR_HIP;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *ws = p;
    return MAMBA_OK;
}

}  // namespace

extern "C" int ssm_scan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int dstate,
                                    int dtype, const void* x, const void* delta, const float* A,
                                    const void* B, const void* C, const float* D, const void* z,
                                    const float* h0, void* y, float* hL,
                                    const mamba_scan_options* options,
                                    const mamba_scan_plan* plan, hipStream_t stream) {
    return mamba::scan_fwd_call(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, D, z, h0,
                                y, hL, options, plan, nullptr, 0, &device_scratch, stream);
}
