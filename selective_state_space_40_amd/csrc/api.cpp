// C ABI of the selective-scan library: argument checks, the chunk plan and
// error mapping around the HIP kernels of scan_kernels.hip.
//
// Every check runs on the host before any HIP call, so a rejected call
// queues nothing and leaves the device untouched. The only HIP calls outside
// the launches are the device and compute-unit-count queries of the
// automatic chunk plan.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <stdint.h>

#include "internal.h"
#include "mamba_scan.h"

namespace {

using mamba::ScanPlan;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet

// Compute units of the current device (cached per device).
int current_cu_count(int* cu) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MAMBA_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) {
        const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
        if (cached > 0) {
            *cu = cached;
            return MAMBA_OK;
        }
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return MAMBA_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
    *cu = n;
    return MAMBA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int dtype,
                int64_t chunk_len) {
    if (batch < 0 || seqlen < 0 || dim < 0 || chunk_len < 0) return MAMBA_ERR_INVALID_ARG;
    if (dtype != MAMBA_DTYPE_F32 && dtype != MAMBA_DTYPE_BF16) return MAMBA_ERR_INVALID_ARG;
    if (dstate < 1 || dstate > MAMBA_SCAN_MAX_DSTATE) return MAMBA_ERR_UNSUPPORTED;
    // every element and workgroup index must fit comfortably in int64 / the grid
    const int64_t lim = int64_t(1) << 48;
    if (batch > lim || seqlen > lim || dim > lim) return MAMBA_ERR_UNSUPPORTED;
    // the (batch, dim, dstate) state and the decode grid stay far from overflow
    if (batch != 0 && dim > (int64_t(1) << 36) / batch) return MAMBA_ERR_UNSUPPORTED;
    if (batch != 0 && dim != 0 && seqlen != 0) {
        if (seqlen > lim / batch || batch * seqlen > lim / dim) return MAMBA_ERR_UNSUPPORTED;
    }
    return MAMBA_OK;
}

// Work decomposition. One wave scans 64 channels of one batch row over one
// chunk. The chunk count is picked so the launch holds about four waves per
// SIMD (four SIMDs per compute unit), which the register budget of the scan
// kernels allows; chunks are never shorter than kMinChunk tokens, since each
// extra chunk costs a summary pass over its tokens.
constexpr int64_t kWavesPerSimdTarget = 4;
constexpr int64_t kMinChunk = 64;

int make_plan(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int64_t chunk_len,
              ScanPlan* plan) {
    if (seqlen == 0 || batch == 0 || dim == 0) {
        plan->chunk_len = seqlen;
        plan->nchunks = 1;
        plan->workspace_bytes = 0;
        return MAMBA_OK;
    }
    int64_t len = chunk_len;
    if (len == 0) {
        int cu = 0;
        const int st = current_cu_count(&cu);
        if (st != MAMBA_OK) return st;
        const int64_t waves = batch * ((dim + mamba::kWave - 1) / mamba::kWave);
        const int64_t target = int64_t(cu) * 4 * kWavesPerSimdTarget;
        int64_t n = (target + waves / 2) / waves;
        const int64_t nmax = seqlen / kMinChunk;
        if (n > nmax) n = nmax;
        if (n < 1) n = 1;
        len = (seqlen + n - 1) / n;
        len = (len + mamba::kTokenTile - 1) / mamba::kTokenTile * mamba::kTokenTile;
    }
    if (len > seqlen) len = seqlen;
    // a chunk's x/delta/z/y rows are addressed with 32-bit byte offsets
    const int64_t esz = 4;  // the wider I/O dtype, so the bound holds for both
    const int64_t max_len = ((int64_t(1) << 32) - 1) / (dim * esz);
    if (max_len < 1) return MAMBA_ERR_UNSUPPORTED;
    if (len > max_len) len = max_len;
    const int64_t nchunks = (seqlen + len - 1) / len;
    const int64_t nblk_d = (dim + mamba::kWave - 1) / mamba::kWave;
    if (nblk_d > (int64_t(1) << 31) / (nchunks * batch)) return MAMBA_ERR_UNSUPPORTED;
    plan->chunk_len = len;
    plan->nchunks = nchunks;
    plan->workspace_bytes = mamba::scan_workspace_bytes(batch, dim, dstate, nchunks);
    return MAMBA_OK;
}

}  // namespace

extern "C" {

int ssm_scan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int dstate,
                                int dtype, int64_t chunk_len, size_t* bytes) {
    if (bytes == nullptr) return MAMBA_ERR_INVALID_ARG;
    const int st = check_shape(batch, seqlen, dim, dstate, dtype, chunk_len);
    if (st != MAMBA_OK) return st;
    ScanPlan plan;
    const int ps = make_plan(batch, seqlen, dim, dstate, chunk_len, &plan);
    if (ps != MAMBA_OK) return ps;
    *bytes = plan.workspace_bytes;
    return MAMBA_OK;
}

int ssm_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int dtype,
                 const void* x, const void* delta, const float* A, const void* B,
                 const void* C, const float* D, const void* z, const float* h0, void* y,
                 float* hL, int64_t chunk_len, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
    int st = check_shape(batch, seqlen, dim, dstate, dtype, chunk_len);
    if (st != MAMBA_OK) return st;
    if (batch == 0 || dim == 0) return MAMBA_OK;
    if (A == nullptr) return MAMBA_ERR_INVALID_ARG;
    if (seqlen > 0 && (x == nullptr || delta == nullptr || B == nullptr || C == nullptr ||
                       y == nullptr))
        return MAMBA_ERR_INVALID_ARG;
    const void* ptrs[] = {x, delta, A, B, C, D, z, h0, y, hL, workspace};
    for (const void* p : ptrs)
        if (p != nullptr && !aligned16(p)) return MAMBA_ERR_MISALIGNED;
    if (seqlen == 0 && hL == nullptr) return MAMBA_OK;

    ScanPlan plan;
    st = make_plan(batch, seqlen, dim, dstate, chunk_len, &plan);
    if (st != MAMBA_OK) return st;
    if (plan.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.workspace_bytes))
        return MAMBA_ERR_WORKSPACE;

    mamba::ScanArgs a;
    a.batch = batch;
    a.seqlen = seqlen;
    a.dim = dim;
    a.dstate = dstate;
    a.io = dtype == MAMBA_DTYPE_F32 ? mamba::kIoF32 : mamba::kIoBF16;
    a.x = x;
    a.delta = delta;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.z = z;
    a.h0 = h0;
    a.y = y;
    a.hL = hL;
    return mamba::launch_scan(a, plan, workspace, stream) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

int ssm_state_update(int64_t batch, int64_t dim, int dstate, int dtype, float* h,
                     const void* x, const void* delta, const float* A, const void* B,
                     const void* C, const float* D, const void* z, void* y,
                     hipStream_t stream) {
    int st = check_shape(batch, 1, dim, dstate, dtype, 0);
    if (st != MAMBA_OK) return st;
    if (batch == 0 || dim == 0) return MAMBA_OK;
    if (h == nullptr || x == nullptr || delta == nullptr || A == nullptr || B == nullptr ||
        C == nullptr || y == nullptr)
        return MAMBA_ERR_INVALID_ARG;
    const void* ptrs[] = {h, x, delta, A, B, C, D, z, y};
    for (const void* p : ptrs)
        if (p != nullptr && !aligned16(p)) return MAMBA_ERR_MISALIGNED;

    mamba::DecodeArgs a;
    a.batch = batch;
    a.dim = dim;
    a.dstate = dstate;
    a.io = dtype == MAMBA_DTYPE_F32 ? mamba::kIoF32 : mamba::kIoBF16;
    a.h = h;
    a.x = x;
    a.delta = delta;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.z = z;
    a.y = y;
    return mamba::launch_state_update(a, stream) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

const char* mamba_status_string(int status) {
    switch (status) {
        case MAMBA_OK: return "MAMBA_OK: success";
        case MAMBA_ERR_INVALID_ARG: return "MAMBA_ERR_INVALID_ARG: invalid argument";
        case MAMBA_ERR_UNSUPPORTED: return "MAMBA_ERR_UNSUPPORTED: unsupported size or dstate";
        case MAMBA_ERR_MISALIGNED: return "MAMBA_ERR_MISALIGNED: pointer not 16-byte aligned";
        case MAMBA_ERR_WORKSPACE: return "MAMBA_ERR_WORKSPACE: workspace missing or too small";
        case MAMBA_ERR_HIP: return "MAMBA_ERR_HIP: HIP runtime error";
        default: return "unknown mamba_status";
    }
}

}  // extern "C"
