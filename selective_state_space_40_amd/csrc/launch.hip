// Single-token decode kernel, the seqlen == 0 state copy, and the entry
// points of internal.h that pick a compiled scan variant.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace mamba {
namespace {

// seqlen == 0: hL = h0 (or zeros).
__global__ __launch_bounds__(256) void state_init_kernel(int64_t count, const float* h0,
                                                         float* hL) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
         i += stride)
        hL[i] = h0 != nullptr ? h0[i] : 0.0f;
}

// ---------------------------------------------------------------------------
// Single-token update. G lanes share one (b, d) and hold S = N / G states
// each, so the fp32 state row of N floats is read and written as G
// contiguous pieces and a wave's accesses are dense. The partial readouts
// are summed across the G lanes with DPP moves inside a quad.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (G == 1) {
        return v;
    } else {
        static_assert(G == 4, "groups of 1 or 4 lanes");
        // quad_perm [1,0,3,2] then [2,3,0,1]
        v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
        v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
        return v;
    }
}

typedef float v4f __attribute__((ext_vector_type(4)));

template <int N, int G, int IO, bool HAS_D, bool HAS_Z>
__global__ __launch_bounds__(256) void state_update_kernel(DecodeArgs a) {
    constexpr int S = N / G;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t pairs = a.batch * a.dim;
    const int64_t p_raw = gid / G;
    const int part = static_cast<int>(gid % G);
    const bool live = p_raw < pairs;
    const int64_t p = live ? p_raw : pairs - 1;
    const int64_t b = p / a.dim;
    const int64_t d = p - b * a.dim;

    float hv[S], Av[S], Bv[S], Cv[S];
    float* hrow = a.h + p * N + part * S;
    const float* arow = a.A + d * N + part * S;
    if constexpr (S == 4) {
        // the state streams through once per step: non-temporal loads and
        // stores keep it from displacing cached data (5% faster for 64
        // layers of 256 x 5120 x 16)
        const v4f hn = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(hrow));
        const float4 h4 = make_float4(hn.x, hn.y, hn.z, hn.w);
        const float4 a4 = *reinterpret_cast<const float4*>(arow);
        hv[0] = h4.x; hv[1] = h4.y; hv[2] = h4.z; hv[3] = h4.w;
        Av[0] = a4.x; Av[1] = a4.y; Av[2] = a4.z; Av[3] = a4.w;
    } else {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            hv[s] = hrow[s];
            Av[s] = arow[s];
        }
    }
    const int64_t brow = b * N + part * S;
    if constexpr (IO == kIoBF16 && S == 4) {
        const uint2 bw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.B) + brow);
        const uint2 cw = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.C) + brow);
        Bv[0] = __uint_as_float(bw.x << 16); Bv[1] = __uint_as_float(bw.x & 0xffff0000u);
        Bv[2] = __uint_as_float(bw.y << 16); Bv[3] = __uint_as_float(bw.y & 0xffff0000u);
        Cv[0] = __uint_as_float(cw.x << 16); Cv[1] = __uint_as_float(cw.x & 0xffff0000u);
        Cv[2] = __uint_as_float(cw.y << 16); Cv[3] = __uint_as_float(cw.y & 0xffff0000u);
    } else {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            Bv[s] = raw_to_f32<IO>(load_raw<IO>(a.B, brow + s));
            Cv[s] = raw_to_f32<IO>(load_raw<IO>(a.C, brow + s));
        }
    }
    // The per-channel inputs are loaded next to the others, before any
    // loaded value is used, so the whole update waits for memory once.
    const uint32_t draw = load_raw<IO>(a.delta, p);
    const uint32_t xraw = load_raw<IO>(a.x, p);
    const uint32_t zraw = HAS_Z ? load_raw<IO>(a.z, p) : 0u;
    const float dskip = HAS_D ? a.D[d] : 0.0f;
    float dbias = 0.0f;
    if (a.delta_bias != nullptr) dbias = a.delta_bias[d];
    float dt = raw_to_f32<IO>(draw) + dbias;
    if (a.delta_softplus) dt = softplus_f32(dt);
    const float u = raw_to_f32<IO>(xraw);
    const float du = dt * u;
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const float e = fast_exp2(dt * (Av[s] * kLog2e));
        hv[s] = fmaf(e, hv[s], du * Bv[s]);
        acc = fmaf(Cv[s], hv[s], acc);
    }
    acc = group_sum<G>(acc);
    if constexpr (HAS_D) acc = fmaf(dskip, u, acc);
    if constexpr (HAS_Z) acc *= silu(raw_to_f32<IO>(zraw));
    // Finish y here: left to itself the compiler sinks the D and z loads
    // into the store branch below, after the other loads have been waited
    // for, which costs a second trip to memory. An empty asm that reads and
    // writes acc pins its computation above the branch.
    asm volatile("" : "+v"(acc));
    if (live) {
        if constexpr (S == 4) {
            const v4f hn = {hv[0], hv[1], hv[2], hv[3]};
            __builtin_nontemporal_store(hn, reinterpret_cast<v4f*>(hrow));
        } else {
#pragma unroll
            for (int s = 0; s < S; ++s) hrow[s] = hv[s];
        }
        if (part == 0) store_io<IO>(a.y, p, acc);
    }
}

template <int N, int IO>
hipError_t launch_decode_n(const DecodeArgs& a, hipStream_t s) {
    constexpr int G = (N % 4 == 0) ? 4 : 1;
    const int64_t lanes = a.batch * a.dim * G;
    const int64_t blocks = (lanes + 255) / 256;
    const bool has_d = a.D != nullptr, has_z = a.z != nullptr;
    if (has_d && has_z)
        hipLaunchKernelGGL((state_update_kernel<N, G, IO, true, true>), dim3(blocks), dim3(256), 0, s, a);
    else if (has_d)
        hipLaunchKernelGGL((state_update_kernel<N, G, IO, true, false>), dim3(blocks), dim3(256), 0, s, a);
    else if (has_z)
        hipLaunchKernelGGL((state_update_kernel<N, G, IO, false, true>), dim3(blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((state_update_kernel<N, G, IO, false, false>), dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int IO>
hipError_t dispatch_decode(const DecodeArgs& a, hipStream_t s) {
    switch (a.dstate) {
#define MAMBA_CASE(n) case n: return launch_decode_n<n, IO>(a, s);
        MAMBA_CASE(1) MAMBA_CASE(2) MAMBA_CASE(3) MAMBA_CASE(4) MAMBA_CASE(5) MAMBA_CASE(6)
        MAMBA_CASE(7) MAMBA_CASE(8) MAMBA_CASE(9) MAMBA_CASE(10) MAMBA_CASE(11) MAMBA_CASE(12)
        MAMBA_CASE(13) MAMBA_CASE(14) MAMBA_CASE(15) MAMBA_CASE(16)
#undef MAMBA_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t scan_workspace_bytes(int64_t batch, int64_t dim, int dstate, int64_t nchunks) {
    if (nchunks <= 1) return 0;
    return static_cast<size_t>(3) * static_cast<size_t>(nchunks) * static_cast<size_t>(batch) *
           static_cast<size_t>(dim) * static_cast<size_t>(dstate) * sizeof(float);
}

hipError_t launch_scan(const ScanArgs& a, const ScanPlan& plan, void* workspace,
                       hipStream_t stream) {
    if (a.seqlen == 0) {
        if (a.hL == nullptr) return hipSuccess;
        const int64_t count = a.batch * a.dim * a.dstate;
        hipLaunchKernelGGL(state_init_kernel, dim3(stride_blocks(count)), dim3(256), 0, stream,
                           count, a.h0, a.hL);
        return hipGetLastError();
    }
    const bool sp = a.delta_softplus != 0;
    if (a.dstate <= 8) {
        if (a.io == kIoF32)
            return sp ? launch_scan_variant<kIoF32, true, 0>(a, plan, workspace, stream)
                      : launch_scan_variant<kIoF32, false, 0>(a, plan, workspace, stream);
        return sp ? launch_scan_variant<kIoBF16, true, 0>(a, plan, workspace, stream)
                  : launch_scan_variant<kIoBF16, false, 0>(a, plan, workspace, stream);
    }
    if (a.io == kIoF32)
        return sp ? launch_scan_variant<kIoF32, true, 1>(a, plan, workspace, stream)
                  : launch_scan_variant<kIoF32, false, 1>(a, plan, workspace, stream);
    return sp ? launch_scan_variant<kIoBF16, true, 1>(a, plan, workspace, stream)
              : launch_scan_variant<kIoBF16, false, 1>(a, plan, workspace, stream);
}

hipError_t launch_state_update(const DecodeArgs& a, hipStream_t stream) {
    return a.io == kIoF32 ? dispatch_decode<kIoF32>(a, stream)
                          : dispatch_decode<kIoBF16>(a, stream);
}

}  // namespace mamba
