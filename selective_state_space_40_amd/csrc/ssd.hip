// Mamba-2's state space dual form on the matrix cores (page "Mamba and State
// Space Models", world.lapla.si, section "Mamba-2: Two Algorithms"). With one
// decay factor exp(dt a_h) per head, a chunk of Q tokens maps its input to
// its output through one lower-triangular matrix, so the chunk is done with
// matrix products and only the state (P x N per head) passes from chunk to
// chunk. Per chunk, with S_i = a * sum_{t <= i} dt_t inside the chunk:
//     G      = C B^T                                   (Q x Q, over N)
//     M[i,j] = G[i,j] exp(S_i - S_j) dt_j for j <= i, 0 above the diagonal
//     Y      = M X + diag(exp(S_i)) C H^T              (Q x P)
//     H     <- exp(S_last) H + (X * w)^T B,  w_j = exp(S_last - S_j) dt_j
//     y      = (Y + D x) * silu(z)
// All four products are bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32
// accumulation.
//
// Work mapping. One workgroup of 4 waves per (batch row, head) walks the
// chunks in order, so the state never leaves the chip: it lives in the MFMA
// accumulators, each wave holding a 32 x N/2 block of it in fp32, and is
// rounded to bf16 in LDS only as the operand of C H^T. Each chunk's x, B and
// C are staged once in LDS (rows padded by 16 bytes against bank conflicts)
// and feed every product; wave w computes the (w/2, w%2) 32 x 32 block of G
// (the block above the diagonal is zero and skipped), of Y, and its block of
// the state update. The matrix M goes through LDS to change from the
// accumulator layout to the operand layout. bf16 I/O, head size 64,
// N = 64 or 128, Q = 64.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace mamba {
namespace {

constexpr int kQ = 64;   // tokens per chunk
constexpr int kP = 64;   // channels per head
constexpr int kSsdThreads = 256;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

template <int N>
struct SsdLds {
    static constexpr int kRowN = N + 8;   // padded row of N bf16
    static constexpr int kRowQ = kQ + 8;  // padded row of 64 bf16
    __bf16 C[kQ][kRowN];    // C rows of the chunk (i, n)
    __bf16 B[kQ][kRowN];    // B rows (j, n)
    __bf16 X[kQ][kRowQ];    // x of the head (j, p)
    __bf16 Xw[kQ][kRowQ];   // x * w_j (j, p)
    __bf16 M[kQ][kRowQ];    // the chunk's matrix (i, j)
    __bf16 H[kP][kRowN];    // the state entering the chunk (p, n)
    float dt[kQ];           // the step as used
    float S[kQ];            // a * running sum of dt inside the chunk
};

__device__ __forceinline__ bf16x8 load8(const __bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// 8 values down a column of a row-major LDS array (k rows apart)
__device__ __forceinline__ bf16x8 load8_col(const __bf16* p, int stride) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = p[e * stride];
    return v;
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of element v of a lane's 32 x 32 accumulator block (its column is
// lane % 32).
__device__ __forceinline__ int acc_row(int v, int lane) {
    return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

template <int N, bool SP, bool HAS_D, bool HAS_Z>
__global__ __launch_bounds__(kSsdThreads) void ssd_fwd_kernel(SsdArgs a) {
    constexpr int NT = N / 64;  // 32 x 32 state blocks per wave
    __shared__ __attribute__((aligned(16))) SsdLds<N> lds;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int64_t b = blockIdx.x / a.nheads;
    const int64_t hd = blockIdx.x - b * a.nheads;
    const int64_t L = a.seqlen;
    const int64_t dim = a.nheads * kP;
    const float alog2 = a.A[hd] * kLog2e;   // log2 of the decay per unit of dt
    const float bias = a.dt_bias != nullptr ? a.dt_bias[hd] : 0.0f;

    // the wave's blocks: rows r0 of G and Y, columns c0 of G (j) and Y (p);
    // state rows p0, columns n0 + 32 t
    const int r0 = 32 * (w >> 1), c0 = 32 * (w & 1);
    const int p0 = 32 * (w >> 1), n0 = (N / 2) * (w & 1);
    const int col = lane & 31;

    f32x16 H[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int p = p0 + acc_row(v, lane), n = n0 + 32 * t + col;
            H[t][v] = a.h0 != nullptr ? a.h0[((b * a.nheads + hd) * kP + p) * N + n] : 0.0f;
        }
    }

    const int64_t nchunks = (L + kQ - 1) / kQ;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * kQ;
        const int cnt = static_cast<int>(min<int64_t>(kQ, L - t0));

        // (1) stage x, B, C of the chunk (tokens past the end as zeros) and
        // the steps with their running sum
        for (int e = tid; e < kQ * (kP / 8); e += kSsdThreads) {
            const int j = e / (kP / 8), q = e - j * (kP / 8);
            uint4 v = make_uint4(0, 0, 0, 0);
            if (j < cnt)
                v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) +
                                                    (b * L + t0 + j) * dim + hd * kP + 8 * q);
            *reinterpret_cast<uint4*>(&lds.X[j][8 * q]) = v;
        }
        for (int e = tid; e < 2 * kQ * (N / 8); e += kSsdThreads) {
            const int which = e / (kQ * (N / 8));
            const int r = e - which * kQ * (N / 8);
            const int j = r / (N / 8), q = r - j * (N / 8);
            uint4 v = make_uint4(0, 0, 0, 0);
            if (j < cnt)
                v = *reinterpret_cast<const uint4*>(
                    static_cast<const uint16_t*>(which ? a.C : a.B) + (b * L + t0 + j) * N + 8 * q);
            *reinterpret_cast<uint4*>(which ? &lds.C[j][8 * q] : &lds.B[j][8 * q]) = v;
        }
        if (w == 0) {
            float dtv = 0.0f;
            if (lane < cnt) {
                const float v = raw_to_f32<kIoBF16>(
                    load_raw<kIoBF16>(a.dt, (b * L + t0 + lane) * a.nheads + hd)) + bias;
                dtv = SP ? softplus_f32(v) : v;
            }
            float s = dtv;  // inclusive running sum over the chunk's lanes
#pragma unroll
            for (int k = 1; k < kWave; k *= 2) {
                const float o = __shfl_up(s, k, kWave);
                if (lane >= k) s += o;
            }
            lds.dt[lane] = dtv;
            lds.S[lane] = s * alog2;  // log2 of the decay from chunk start through token lane
        }
        __syncthreads();

        // (2) x * w_j, the state as bf16, and the wave's block of M
        const float s_last = lds.S[kQ - 1];
        for (int e = tid; e < kQ * kP; e += kSsdThreads) {
            const int j = e / kP, p = e - j * kP;
            const float wj = fast_exp2(s_last - lds.S[j]) * lds.dt[j];
            lds.Xw[j][p] = static_cast<__bf16>(static_cast<float>(lds.X[j][p]) * wj);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                lds.H[p0 + acc_row(v, lane)][n0 + 32 * t + col] = static_cast<__bf16>(H[t][v]);
        if (r0 >= c0) {  // the block above the diagonal is zero
            f32x16 G = {};
#pragma unroll
            for (int k = 0; k < N; k += 16) {
                const int kk = k + 8 * (lane >> 5);
                G = mfma(load8(&lds.C[r0 + col][kk]), load8(&lds.B[c0 + col][kk]), G);
            }
            const int j = c0 + col;
            const float sj = lds.S[j], dtj = lds.dt[j];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int i = r0 + acc_row(v, lane);
                const float m = i >= j ? G[v] * fast_exp2(lds.S[i] - sj) * dtj : 0.0f;
                lds.M[i][j] = static_cast<__bf16>(m);
            }
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) lds.M[r0 + acc_row(v, lane)][c0 + col] = static_cast<__bf16>(0.0f);
        }
        __syncthreads();

        // (3) the wave's block of Y: M X (only j <= last row of the block)
        // plus diag(exp(S)) C H^T; then skip, gate and store
        {
            f32x16 Yd = {}, Yo = {};
            const int kmax = r0 + 32;
            for (int k = 0; k < kmax; k += 16) {
                const int kk = k + 8 * (lane >> 5);
                Yd = mfma(load8(&lds.M[r0 + col][kk]), load8_col(&lds.X[kk][c0 + col], SsdLds<N>::kRowQ), Yd);
            }
#pragma unroll
            for (int k = 0; k < N; k += 16) {
                const int kk = k + 8 * (lane >> 5);
                Yo = mfma(load8(&lds.C[r0 + col][kk]), load8(&lds.H[c0 + col][kk]), Yo);
            }
            const int p = c0 + col;
            const int64_t chan = hd * kP + p;
            const float dskip = HAS_D ? a.D[chan] : 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int i = r0 + acc_row(v, lane);
                if (i < cnt) {
                    float out = Yd[v] + fast_exp2(lds.S[i]) * Yo[v];
                    const int64_t idx = (b * L + t0 + i) * dim + chan;
                    if constexpr (HAS_D) out = fmaf(dskip, static_cast<float>(lds.X[i][p]), out);
                    if constexpr (HAS_Z) out *= silu(raw_to_f32<kIoBF16>(load_raw<kIoBF16>(a.z, idx)));
                    store_io<kIoBF16>(a.y, idx, out);
                }
            }
        }

        // (4) the state: H <- exp(S_last) H + (X w)^T B
        {
            const float decay = fast_exp2(s_last);
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int v = 0; v < 16; ++v) H[t][v] *= decay;
#pragma unroll
            for (int k = 0; k < kQ; k += 16) {
                const int kk = k + 8 * (lane >> 5);
                const bf16x8 xa = load8_col(&lds.Xw[kk][p0 + col], SsdLds<N>::kRowQ);
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    H[t] = mfma(xa, load8_col(&lds.B[kk][n0 + 32 * t + col], SsdLds<N>::kRowN), H[t]);
            }
        }
        __syncthreads();
    }

    if (a.hL != nullptr) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int p = p0 + acc_row(v, lane), n = n0 + 32 * t + col;
                a.hL[((b * a.nheads + hd) * kP + p) * N + n] = H[t][v];
            }
    }
}

// seqlen == 0: hL = h0 (or zeros).
__global__ __launch_bounds__(256) void ssd_state_copy_kernel(int64_t count, const float* h0,
                                                             float* hL) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
         i += stride)
        hL[i] = h0 != nullptr ? h0[i] : 0.0f;
}

template <int N, bool SP>
hipError_t launch_ssd_n(const SsdArgs& a, hipStream_t s) {
    const dim3 grid(a.batch * a.nheads), block(kSsdThreads);
    const bool has_d = a.D != nullptr, has_z = a.z != nullptr;
    if (has_d && has_z) hipLaunchKernelGGL((ssd_fwd_kernel<N, SP, true, true>), grid, block, 0, s, a);
    else if (has_d) hipLaunchKernelGGL((ssd_fwd_kernel<N, SP, true, false>), grid, block, 0, s, a);
    else if (has_z) hipLaunchKernelGGL((ssd_fwd_kernel<N, SP, false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((ssd_fwd_kernel<N, SP, false, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ssd_fwd(const SsdArgs& a, hipStream_t stream) {
    if (a.seqlen == 0) {
        if (a.hL == nullptr) return hipSuccess;
        const int64_t count = a.batch * a.nheads * kP * a.dstate;
        hipLaunchKernelGGL(ssd_state_copy_kernel, dim3(stride_blocks(count)), dim3(256), 0, stream,
                           count, a.h0, a.hL);
        return hipGetLastError();
    }
    const bool sp = a.dt_softplus != 0;
    if (a.dstate == 64) return sp ? launch_ssd_n<64, true>(a, stream) : launch_ssd_n<64, false>(a, stream);
    if (a.dstate == 128) return sp ? launch_ssd_n<128, true>(a, stream) : launch_ssd_n<128, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace mamba
