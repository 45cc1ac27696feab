// Short causal depthwise convolution of the Mamba block and its decode step
// (page "Mamba and State Space Models", world.lapla.si, section "A State of
// Fixed Size": next to its SSM state each channel keeps the last 4 inputs of
// a short convolution). Per batch row b, channel d, token t, width W:
//     pre[b,t,d] = bias[d] + sum_{k<W} weight[d,k] * x[b, t-(W-1)+k, d]
//     y[b,t,d]   = silu(pre) or pre
// Inputs before the first token come from the carried state, the last W
// inputs of the channel (newest last), kept in the I/O dtype since they are
// inputs and so exact in it.
//
// Work mapping. The convolution is HBM-bound (about 2 I/O elements moved per
// 2W+6 lane-ops) and elementwise across channels, so a thread owns VEC = 4
// adjacent channels (one 8-byte bf16 or 16-byte fp32 access per row) and
// kConvTokens consecutive tokens. It loads its W-1 halo rows and its own rows
// all at once, before using any of them, so one trip to memory covers the
// thread's whole window; the halo rows are the previous thread's last rows
// and come from L2. Lanes run along the channels, so a wave's row access is
// 512 contiguous bytes (bf16). Workgroups are numbered so that those of one
// XCD cover one contiguous range of token chunks, so the halo rows are found
// in the XCD's own L2. The thread of the first token chunk of each channel
// group also reads the carried state. The handed-on state is written by the
// thread of the last token chunk, which holds the last W rows, when the
// sequence is a whole number of chunks and the two states are distinct
// buffers; otherwise a second small kernel queued after the first writes it,
// so the states may alias.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace mamba {
namespace {

constexpr int kConvTokens = 16;  // tokens per thread of the forward kernel
constexpr int kConvBlock = 256;
// The decode state streams through once per step: non-temporal loads and
// stores keep it from displacing cached data (64 layers of 256 x 5120, W=4:
// 461 us against 523 us with ordinary accesses).
constexpr bool kConvStateNt = true;
// The output of the whole-sequence convolution is written once and not
// read back by this kernel: non-temporal stores (64.3 us against 68.1 us
// for the Mamba-2.8B layer input).
constexpr bool kConvYNt = true;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

// Word loads and stores, non-temporal when NT (data that streams through
// once and should not displace cached data).
template <bool NT, typename T>
__device__ __forceinline__ T ld_words(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT, typename T>
__device__ __forceinline__ void st_words(T v, T* p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// K consecutive I/O elements held as raw 32-bit words and moved with the
// widest accesses their size allows (callers guarantee that alignment).
template <int IO, int K>
struct Run {
    static constexpr int kBytes = K * (IO == kIoF32 ? 4 : 2);
    static constexpr bool kWords = kBytes % 4 == 0;
    static constexpr int kN = kWords ? kBytes / 4 : K;  // words, or single elements
    uint32_t w[kN];

    template <bool NT = false>
    __device__ __forceinline__ void load(const void* base, int64_t elem) {
        if constexpr (!kWords) {
#pragma unroll
            for (int e = 0; e < K; ++e) w[e] = load_raw<IO>(base, elem + e);
        } else {
            const char* p = static_cast<const char*>(base) + elem * (IO == kIoF32 ? 4 : 2);
            if constexpr (kBytes % 16 == 0) {
#pragma unroll
                for (int q = 0; q < kN / 4; ++q) {
                    const v4u v = ld_words<NT>(reinterpret_cast<const v4u*>(p) + q);
                    w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
                }
            } else if constexpr (kBytes % 8 == 0) {
#pragma unroll
                for (int q = 0; q < kN / 2; ++q) {
                    const v2u v = ld_words<NT>(reinterpret_cast<const v2u*>(p) + q);
                    w[2 * q] = v.x; w[2 * q + 1] = v.y;
                }
            } else {
#pragma unroll
                for (int q = 0; q < kN; ++q) w[q] = ld_words<NT>(reinterpret_cast<const uint32_t*>(p) + q);
            }
        }
    }

    template <bool NT = false>
    __device__ __forceinline__ void store(void* base, int64_t elem) const {
        if constexpr (!kWords) {
#pragma unroll
            for (int e = 0; e < K; ++e) {
                if constexpr (IO == kIoF32)
                    static_cast<uint32_t*>(base)[elem + e] = w[e];
                else
                    static_cast<uint16_t*>(base)[elem + e] = static_cast<uint16_t>(w[e]);
            }
        } else {
            char* p = static_cast<char*>(base) + elem * (IO == kIoF32 ? 4 : 2);
            if constexpr (kBytes % 16 == 0) {
#pragma unroll
                for (int q = 0; q < kN / 4; ++q)
                    st_words<NT>(v4u{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]},
                                 reinterpret_cast<v4u*>(p) + q);
            } else if constexpr (kBytes % 8 == 0) {
#pragma unroll
                for (int q = 0; q < kN / 2; ++q)
                    st_words<NT>(v2u{w[2 * q], w[2 * q + 1]}, reinterpret_cast<v2u*>(p) + q);
            } else {
#pragma unroll
                for (int q = 0; q < kN; ++q) st_words<NT>(w[q], reinterpret_cast<uint32_t*>(p) + q);
            }
        }
    }

    // raw bits of element e (bf16: in the low 16 bits)
    __device__ __forceinline__ uint32_t get(int e) const {
        if constexpr (IO == kIoF32 || !kWords) return w[e];
        else return (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
    }

    __device__ __forceinline__ void set(int e, uint32_t bits) {
        if constexpr (IO == kIoF32 || !kWords) {
            w[e] = bits;
        } else {
            const int s = 16 * (e & 1);
            w[e >> 1] = (w[e >> 1] & ~(0xffffu << s)) | ((bits & 0xffffu) << s);
        }
    }

    __device__ __forceinline__ float f32(int e) const {
        const uint32_t r = get(e);
        if constexpr (IO == kIoF32) return __uint_as_float(r);
        else return __uint_as_float(r << 16);
    }
};

// fp32 -> raw I/O bits, bf16 rounded to nearest even
template <int IO>
__device__ __forceinline__ uint32_t to_raw(float v) {
    if constexpr (IO == kIoF32) return __float_as_uint(v);
    else return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

template <int W, int VEC>
__device__ __forceinline__ void load_taps(const ConvArgs& a, int64_t c0, float (&wt)[VEC][W],
                                          float (&bs)[VEC]) {
    // weight rows of VEC adjacent channels are VEC*W contiguous floats; when
    // VEC*W is a multiple of 4 they start 16-byte aligned (the weight pointer
    // is, and c0*W is a multiple of VEC*W), and likewise the bias run
    if constexpr ((VEC * W) % 4 == 0) {
        const float4* wp = reinterpret_cast<const float4*>(a.weight + c0 * W);
#pragma unroll
        for (int q = 0; q < VEC * W / 4; ++q) {
            const float4 v = wp[q];
            const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) wt[(4 * q + u) / W][(4 * q + u) % W] = e[u];
        }
    } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v)
#pragma unroll
            for (int k = 0; k < W; ++k) wt[v][k] = a.weight[(c0 + v) * W + k];
    }
    if constexpr (VEC % 4 == 0) {
#pragma unroll
        for (int q = 0; q < VEC / 4; ++q) {
            const float4 v = a.bias != nullptr ? reinterpret_cast<const float4*>(a.bias + c0)[q]
                                               : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            bs[4 * q] = v.x; bs[4 * q + 1] = v.y; bs[4 * q + 2] = v.z; bs[4 * q + 3] = v.w;
        }
    } else if constexpr (VEC % 2 == 0) {
#pragma unroll
        for (int q = 0; q < VEC / 2; ++q) {
            const float2 v = a.bias != nullptr ? reinterpret_cast<const float2*>(a.bias + c0)[q]
                                               : make_float2(0.0f, 0.0f);
            bs[2 * q] = v.x; bs[2 * q + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) bs[v] = a.bias != nullptr ? a.bias[c0 + v] : 0.0f;
    }
}

template <bool SILU>
__device__ __forceinline__ float conv_act(float pre) {
    return SILU ? silu(pre) : pre;
}

template <int W, int IO, int VEC, bool SILU>
__global__ __launch_bounds__(kConvBlock) void conv1d_fwd_kernel(ConvArgs a, int64_t ncg,
                                                                int64_t ntc) {
    constexpr int T = kConvTokens;
    constexpr int R = T + W - 1;  // window rows: W-1 halo rows, then T own rows
    const int64_t blk = xcd_contiguous_block(blockIdx.x, gridDim.x);
    const int64_t gid = blk * kConvBlock + threadIdx.x;
    if (gid >= a.batch * ntc * ncg) return;  // no barriers below: exiting early is safe
    const int64_t cg = gid % ncg;
    const int64_t rest = gid / ncg;
    const int64_t tc = rest % ntc;
    const int64_t b = rest / ntc;
    const int64_t c0 = cg * VEC;
    const int64_t t0 = tc * T;
    const int64_t L = a.seqlen;
    const int64_t row0 = b * L;  // row of token 0 of this batch row

    // Every window row is fetched first. Rows are clamped into the sequence:
    // rows before token 0 are replaced by carried inputs below, rows past
    // the end feed only outputs that are not stored.
    Run<IO, VEC> win[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        int64_t s = t0 - (W - 1) + i;
        s = s < 0 ? 0 : (s > L - 1 ? L - 1 : s);
        win[i].load(a.x, (row0 + s) * a.dim + c0);
    }
    float wt[VEC][W], bs[VEC];
    load_taps<W, VEC>(a, c0, wt, bs);

    if (tc == 0) {
        // Carried inputs of the VEC channels: (b, c, 0..W-1), newest last.
        Run<IO, VEC * W> carried;
        if (a.state_in != nullptr) {
            carried.load(a.state_in, (b * a.dim + c0) * W);
        } else {
#pragma unroll
            for (int q = 0; q < Run<IO, VEC * W>::kN; ++q) carried.w[q] = 0u;
        }
        // window rows before token 0 take the carried inputs
#pragma unroll
        for (int i = 0; i < W - 1; ++i)
#pragma unroll
            for (int v = 0; v < VEC; ++v) win[i].set(v, carried.get(v * W + i + 1));
    }

    // A full chunk stores every token without branches, so the waits for
    // the window stay exact while the stores are in flight; only the last
    // chunk of a sequence that is not a multiple of T takes the guarded path.
    const int64_t nout = L - t0 < T ? L - t0 : T;
    auto token = [&](int j) {
        Run<IO, VEC> o;
#pragma unroll
        for (int q = 0; q < Run<IO, VEC>::kN; ++q) o.w[q] = 0u;
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            float pre = bs[v];
#pragma unroll
            for (int k = 0; k < W; ++k) pre = fmaf(wt[v][k], win[j + k].f32(v), pre);
            o.set(v, to_raw<IO>(conv_act<SILU>(pre)));
        }
        o.template store<kConvYNt>(a.y, (row0 + t0 + j) * a.dim + c0);
    };
    if (nout == T) {
#pragma unroll
        for (int j = 0; j < T; ++j) token(j);
        // the last chunk's rows T-1 .. T+W-2 are the last W inputs
        if (a.fuse_state && tc == ntc - 1) {
            Run<IO, VEC * W> out;
#pragma unroll
            for (int k = 0; k < W; ++k)
#pragma unroll
                for (int v = 0; v < VEC; ++v) out.set(v * W + k, win[T - 1 + k].get(v));
            out.store(a.state_out, (b * a.dim + c0) * W);
        }
    } else {
#pragma unroll
        for (int j = 0; j < T; ++j)
            if (j < nout) token(j);
    }
}

// Decode: the new input joins the carried W inputs (the oldest leaves) and
// one output is produced; the state row of VEC channels (VEC*W elements) is
// read and written in place with wide accesses.
template <int W, int IO, int VEC, bool SILU>
__global__ __launch_bounds__(kConvBlock) void conv1d_update_kernel(ConvArgs a, int64_t ncg) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * kConvBlock + threadIdx.x;
    if (gid >= a.batch * ncg) return;
    const int64_t cg = gid % ncg;
    const int64_t b = gid / ncg;
    const int64_t c0 = cg * VEC;
    Run<IO, VEC * W> st;
    st.template load<kConvStateNt>(a.state_in, (b * a.dim + c0) * W);
    Run<IO, VEC> xin;
    xin.load(a.x, b * a.dim + c0);
    float wt[VEC][W], bs[VEC];
    load_taps<W, VEC>(a, c0, wt, bs);
    Run<IO, VEC> o;
#pragma unroll
    for (int q = 0; q < Run<IO, VEC>::kN; ++q) o.w[q] = 0u;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
#pragma unroll
        for (int k = 0; k < W - 1; ++k) st.set(v * W + k, st.get(v * W + k + 1));
        st.set(v * W + W - 1, xin.get(v));
        float pre = bs[v];
#pragma unroll
        for (int k = 0; k < W; ++k) pre = fmaf(wt[v][k], st.f32(v * W + k), pre);
        o.set(v, to_raw<IO>(conv_act<SILU>(pre)));
    }
    st.template store<kConvStateNt>(a.state_out, (b * a.dim + c0) * W);
    o.store(a.y, b * a.dim + c0);
}

// The handed-on state: per (b, d) the last W inputs of the sequence,
// reaching into the carried ones when the sequence is shorter than W (all
// of them when it is empty). Each thread reads all W values before it
// writes any, and the forward kernel, which also reads the carried state,
// has finished before this one starts, so state_out may alias state_in.
template <int IO>
__global__ __launch_bounds__(kConvBlock) void conv1d_state_out_kernel(ConvArgs a) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kConvBlock;
    const int64_t pairs = a.batch * a.dim;
    const int W = a.width;
    for (int64_t p = static_cast<int64_t>(blockIdx.x) * kConvBlock + threadIdx.x; p < pairs;
         p += stride) {
        const int64_t b = p / a.dim;
        const int64_t d = p - b * a.dim;
        uint32_t v[kConvMaxWidth];
#pragma unroll
        for (int k = 0; k < kConvMaxWidth; ++k) {
            if (k < W) {
                const int64_t s = a.seqlen - W + k;
                if (s >= 0)
                    v[k] = load_raw<IO>(a.x, (b * a.seqlen + s) * a.dim + d);
                else
                    v[k] = a.state_in != nullptr ? load_raw<IO>(a.state_in, p * W + (W + s)) : 0u;
            }
        }
#pragma unroll
        for (int k = 0; k < kConvMaxWidth; ++k) {
            if (k < W) {
                if constexpr (IO == kIoF32)
                    static_cast<uint32_t*>(a.state_out)[p * W + k] = v[k];
                else
                    static_cast<uint16_t*>(a.state_out)[p * W + k] = static_cast<uint16_t>(v[k]);
            }
        }
    }
}

template <int W, int IO, int VEC>
hipError_t launch_conv_wv(const ConvArgs& a, bool update, hipStream_t s) {
    const int64_t ncg = a.dim / VEC;
    if (update) {
        const int64_t blocks = (a.batch * ncg + kConvBlock - 1) / kConvBlock;
        if (a.silu)
            hipLaunchKernelGGL((conv1d_update_kernel<W, IO, VEC, true>), dim3(blocks),
                               dim3(kConvBlock), 0, s, a, ncg);
        else
            hipLaunchKernelGGL((conv1d_update_kernel<W, IO, VEC, false>), dim3(blocks),
                               dim3(kConvBlock), 0, s, a, ncg);
    } else {
        const int64_t ntc = a.seqlen > 0 ? (a.seqlen + kConvTokens - 1) / kConvTokens : 1;
        const int64_t blocks = (a.batch * ntc * ncg + kConvBlock - 1) / kConvBlock;
        if (a.silu)
            hipLaunchKernelGGL((conv1d_fwd_kernel<W, IO, VEC, true>), dim3(blocks),
                               dim3(kConvBlock), 0, s, a, ncg, ntc);
        else
            hipLaunchKernelGGL((conv1d_fwd_kernel<W, IO, VEC, false>), dim3(blocks),
                               dim3(kConvBlock), 0, s, a, ncg, ntc);
    }
    return hipGetLastError();
}

// The decode step moves so few bytes per thread that more threads beat wider
// accesses: 2 channels per thread measured 524.6 us for 64 layers of
// 256 x 5120 against 558.1 (1 channel), 560.1 (4) and 750.3 (8).
template <int W, int IO>
hipError_t launch_conv_w(const ConvArgs& a, bool update, hipStream_t s) {
    if (update)
        return a.dim % 2 == 0 ? launch_conv_wv<W, IO, 2>(a, update, s)
                              : launch_conv_wv<W, IO, 1>(a, update, s);
    return a.dim % 4 == 0 ? launch_conv_wv<W, IO, 4>(a, update, s)
                          : launch_conv_wv<W, IO, 1>(a, update, s);
}

template <int IO>
hipError_t launch_conv_io(const ConvArgs& args, bool update, hipStream_t s) {
    ConvArgs a = args;
    // the forward kernel hands on the state itself when its last chunk holds
    // the last W rows whole and the two states are different buffers
    a.fuse_state = !update && a.state_out != nullptr && a.state_out != a.state_in &&
                   a.seqlen >= a.width && a.seqlen % kConvTokens == 0;
    hipError_t e = hipSuccess;
    if (update || a.seqlen > 0) {
        switch (a.width) {
            case 1: e = launch_conv_w<1, IO>(a, update, s); break;
            case 2: e = launch_conv_w<2, IO>(a, update, s); break;
            case 3: e = launch_conv_w<3, IO>(a, update, s); break;
            case 4: e = launch_conv_w<4, IO>(a, update, s); break;
            default: return hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
    }
    if (!update && a.state_out != nullptr && !a.fuse_state) {
        hipLaunchKernelGGL((conv1d_state_out_kernel<IO>), dim3(stride_blocks(a.batch * a.dim)),
                           dim3(kConvBlock), 0, s, a);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

hipError_t launch_conv1d(const ConvArgs& a, bool update, hipStream_t stream) {
    return a.io == kIoF32 ? launch_conv_io<kIoF32>(a, update, stream)
                          : launch_conv_io<kIoBF16>(a, update, stream);
}

}  // namespace mamba
