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
// All products are bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32
// accumulation.
//
// Work mapping. One workgroup of 4 waves per (batch row, head) walks the
// chunks in order, so the state never leaves the chip: it lives in the MFMA
// accumulators as H^T (N x P), wave w holding rows n of its quarter of N for
// all 64 channels, in fp32; it is rounded to bf16 in LDS only as an operand.
// Wave w owns tokens i in [16w, 16w + 16) of the chunk. It forms G^T for its
// tokens (rows j <= its last token only) and turns it into M^T in its
// accumulators; the accumulator of a 16 x 16 block holds, in each lane, one
// column i and rows j = 4(lane / 16) + 0..3, and two such blocks are exactly
// the K = 32 operand of the next product up to a fixed permutation of K, so
// Y^T = X^T M^T takes M^T straight from the accumulators (X^T is read with
// the same permutation) and M never goes through LDS. The chunk's x, B and C
// are staged once in LDS (rows padded by 16 bytes), B also transposed and
// scaled by w_j for the state update, and the next chunk's inputs are loaded
// into registers while this one is computed. bf16 I/O, head size 64,
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
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

template <int N>
struct SsdLds {
    static constexpr int kRowN = N + 8;   // padded row of N bf16
    static constexpr int kRowQ = kQ + 8;  // padded row of 64 bf16
    __bf16 C[kQ][kRowN];     // C rows of the chunk (i, n)
    __bf16 B[kQ][kRowN];     // B rows (j, n)
    __bf16 Bt[N][kRowQ];     // B transposed (n, j)
    __bf16 Xt[kP][kRowQ];    // x transposed (p, j)
    __bf16 H[kP][kRowN];     // the state entering the chunk (p, n)
    float dt[kQ];            // the step as used
    float S[kQ];             // log2 of the decay from chunk start through token j
    float w[kQ];             // exp(S_last - S_j) dt_j: weight of token j in the state update
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const __bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// Operand whose 8 K values are two runs of 4: p[0..3] and q[0..3].
__device__ __forceinline__ bf16x8 lds4x2(const __bf16* p, const __bf16* q) {
    typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(q);
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = a[e];
        v[e + 4] = b[e];
    }
    return v;
}

// The next chunk's inputs, held in registers between chunks. Threads
// 0 .. 63 each hold an 8 x 8 block (8 tokens, 8 channels) of x, the next
// N threads (N / 8 blocks per 8 tokens) an 8 x 8 block of B; all threads
// hold a share of C.
template <int N>
struct Prefetch {
    static constexpr int kXBlocks = (kQ / 8) * (kP / 8);
    static constexpr int kBBlocks = (kQ / 8) * (N / 8);
    static constexpr int kC = kQ * N / 8 / kSsdThreads;   // uint4 of C per thread
    uint4 blk[8], c[kC];
    float dt;
};

template <int N>
__device__ __forceinline__ void fetch_chunk(const SsdArgs& a, int64_t bb, int64_t hd, int64_t t0,
                                            int cnt, Prefetch<N>& f) {
    const int tid = threadIdx.x;
    const int64_t L = a.seqlen, dim = a.nheads * kP;
    const uint16_t* src = nullptr;
    int64_t stride = 0;
    int jb = 0;
    if (tid < Prefetch<N>::kXBlocks) {
        jb = tid / (kP / 8);
        src = static_cast<const uint16_t*>(a.x) + (bb * L + t0) * dim + hd * kP + 8 * (tid % (kP / 8));
        stride = dim;
    } else if (tid < Prefetch<N>::kXBlocks + Prefetch<N>::kBBlocks) {
        const int e = tid - Prefetch<N>::kXBlocks;
        jb = e / (N / 8);
        src = static_cast<const uint16_t*>(a.B) + (bb * L + t0) * N + 8 * (e % (N / 8));
        stride = N;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int j = 8 * jb + r;
        f.blk[r] = (src != nullptr && j < cnt)
                       ? *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(j) * stride)
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < Prefetch<N>::kC; ++r) {
        const int e = tid + r * kSsdThreads;
        const int j = e / (N / 8), q = e % (N / 8);
        f.c[r] = j < cnt ? *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.C) +
                                                           (bb * L + t0 + j) * N + 8 * q)
                         : make_uint4(0, 0, 0, 0);
    }
    const int lane = tid & (kWave - 1);
    f.dt = (tid < kWave && lane < cnt)
               ? raw_to_f32<kIoBF16>(load_raw<kIoBF16>(a.dt, (bb * L + t0 + lane) * a.nheads + hd))
               : 0.0f;
}

// 8 x 8 bf16 transpose in registers: in[r] holds row r (8 values), out[f]
// column f.
__device__ __forceinline__ void transpose8(const uint4 (&in)[8], uint4 (&out)[8]) {
    uint32_t iw[8][4];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        iw[r][0] = in[r].x; iw[r][1] = in[r].y; iw[r][2] = in[r].z; iw[r][3] = in[r].w;
    }
#pragma unroll
    for (int f = 0; f < 8; ++f) {
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t lo = iw[2 * q][f >> 1], hi = iw[2 * q + 1][f >> 1];
            o[q] = (f & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        out[f] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

template <int N, bool SP, bool HAS_D, bool HAS_Z>
__global__ __launch_bounds__(kSsdThreads) __attribute__((amdgpu_waves_per_eu(2)))
void ssd_fwd_kernel(SsdArgs a) {
    constexpr int NW = N / 4;        // state rows n per wave
    constexpr int NTN = NW / 16;     // 16-row blocks of them
    constexpr int RN = SsdLds<N>::kRowN, RQ = SsdLds<N>::kRowQ;
    __shared__ __attribute__((aligned(16))) SsdLds<N> lds;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane >> 4, c = lane & 15;
    const int64_t bb = blockIdx.x / a.nheads;
    const int64_t hd = blockIdx.x - bb * a.nheads;
    const int64_t L = a.seqlen;
    const int64_t dim = a.nheads * kP;
    const float alog2 = a.A[hd] * kLog2e;
    const float bias = a.dt_bias != nullptr ? a.dt_bias[hd] : 0.0f;
    const int i = 16 * w + c;        // this lane's token of the chunk (as output column)

    // state H^T: block (nt, pt) holds rows n = nw0 + 16 nt + 4 g + v, column p = 16 pt + c
    const int nw0 = NW * w;
    f32x4 H[NTN][4];
#pragma unroll
    for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int n = nw0 + 16 * nt + 4 * g + v, p = 16 * pt + c;
                H[nt][pt][v] = a.h0 != nullptr ? a.h0[((bb * a.nheads + hd) * kP + p) * N + n] : 0.0f;
            }

    const int64_t nchunks = (L + kQ - 1) / kQ;
    Prefetch<N> pf;
    fetch_chunk<N>(a, bb, hd, 0, static_cast<int>(min<int64_t>(kQ, L)), pf);
    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t t0 = ch * kQ;
        const int cnt = static_cast<int>(min<int64_t>(kQ, L - t0));

        // (1) stage the chunk: x transposed, B as it is and transposed, C;
        // the steps, their running sum and the token weights; the state
        // entering the chunk as bf16 (p, n)
        if (tid < Prefetch<N>::kXBlocks + Prefetch<N>::kBBlocks) {
            uint4 tr[8];
            transpose8(pf.blk, tr);
            if (tid < Prefetch<N>::kXBlocks) {
                const int jb = tid / (kP / 8), pb = tid % (kP / 8);
#pragma unroll
                for (int f = 0; f < 8; ++f) *reinterpret_cast<uint4*>(&lds.Xt[8 * pb + f][8 * jb]) = tr[f];
            } else {
                const int e = tid - Prefetch<N>::kXBlocks;
                const int jb = e / (N / 8), nb = e % (N / 8);
#pragma unroll
                for (int f = 0; f < 8; ++f) {
                    *reinterpret_cast<uint4*>(&lds.Bt[8 * nb + f][8 * jb]) = tr[f];
                    *reinterpret_cast<uint4*>(&lds.B[8 * jb + f][8 * nb]) = pf.blk[f];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < Prefetch<N>::kC; ++r) {
            const int e = tid + r * kSsdThreads;
            const int j = e / (N / 8), q = e % (N / 8);
            *reinterpret_cast<uint4*>(&lds.C[j][8 * q]) = pf.c[r];
        }
        if (w == 0) {
            const float v = pf.dt + bias;
            const float dtv = lane < cnt ? (SP ? softplus_f32(v) : v) : 0.0f;
            float s = dtv;
#pragma unroll
            for (int k = 1; k < kWave; k *= 2) {
                const float o = __shfl_up(s, k, kWave);
                if (lane >= k) s += o;
            }
            s *= alog2;
            const float last = __shfl(s, kWave - 1, kWave);
            lds.dt[lane] = dtv;
            lds.S[lane] = s;
            lds.w[lane] = fast_exp2(last - s) * dtv;
        }
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
                bf16x4 hv;
#pragma unroll
                for (int v = 0; v < 4; ++v) hv[v] = static_cast<__bf16>(H[nt][pt][v]);
                *reinterpret_cast<bf16x4*>(&lds.H[16 * pt + c][nw0 + 16 * nt + 4 * g]) = hv;
            }
        __syncthreads();

        // the next chunk's loads go out now and land during this chunk
        if (ch + 1 < nchunks)
            fetch_chunk<N>(a, bb, hd, t0 + kQ, static_cast<int>(min<int64_t>(kQ, L - t0 - kQ)), pf);
        const float s_last = lds.S[kQ - 1];

        // (3) M^T for this wave's tokens: blocks jt = 0 .. w of G^T = B C^T
        f32x4 Mt[4];
        const float si = lds.S[i];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            Mt[jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (jt <= w) {
#pragma unroll
                for (int k = 0; k < N; k += 32)
                    Mt[jt] = mfma16(lds8(&lds.B[16 * jt + c][k + 8 * g]),
                                    lds8(&lds.C[i][k + 8 * g]), Mt[jt]);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int j = 16 * jt + 4 * g + v;
                    Mt[jt][v] = j <= i ? Mt[jt][v] * fast_exp2(si - lds.S[j]) * lds.dt[j] : 0.0f;
                }
            }
        }
        // Y^T = X^T M^T + exp(S_i) H C^T: blocks pt (rows p = 16 pt + 4 g + v, column i)
        f32x4 Yd[4], Yo[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            Yd[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            Yo[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            if (2 * s2 <= w) {
                // K = 32 tokens j: j = 32 s2 + 4 g + e (e < 4) and 32 s2 + 16 + 4 g + (e - 4)
                bf16x8 mb;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    mb[e] = static_cast<__bf16>(Mt[2 * s2][e]);
                    mb[e + 4] = static_cast<__bf16>(Mt[2 * s2 + 1][e]);
                }
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
                    Yd[pt] = mfma16(lds4x2(&lds.Xt[16 * pt + c][32 * s2 + 4 * g],
                                           &lds.Xt[16 * pt + c][32 * s2 + 16 + 4 * g]),
                                    mb, Yd[pt]);
            }
        }
#pragma unroll
        for (int k = 0; k < N; k += 32) {
            const bf16x8 cb = lds8(&lds.C[i][k + 8 * g]);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
                Yo[pt] = mfma16(lds8(&lds.H[16 * pt + c][k + 8 * g]), cb, Yo[pt]);
        }
        if (i < cnt) {
            const float eo = fast_exp2(si);
            const int64_t row = (bb * L + t0 + i) * dim + hd * kP;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int p0 = 16 * pt + 4 * g;
                float out[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    out[v] = fmaf(eo, Yo[pt][v], Yd[pt][v]);
                    if constexpr (HAS_D)
                        out[v] = fmaf(a.D[hd * kP + p0 + v], static_cast<float>(lds.Xt[p0 + v][i]), out[v]);
                }
                if constexpr (HAS_Z) {
                    const uint2 zr = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.z) + row + p0);
                    out[0] *= silu(__uint_as_float(zr.x << 16));
                    out[1] *= silu(__uint_as_float(zr.x & 0xffff0000u));
                    out[2] *= silu(__uint_as_float(zr.y << 16));
                    out[3] *= silu(__uint_as_float(zr.y & 0xffff0000u));
                }
                uint2 o;
                o.x = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(out[0]))) |
                      (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(out[1]))) << 16);
                o.y = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(out[2]))) |
                      (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(out[3]))) << 16);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y) + row + p0) = o;
            }
        }

        // (4) the state: H^T <- exp(S_last) H^T + (B w)^T X, w applied as the
        // operand is read
        const float decay = fast_exp2(s_last);
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                for (int v = 0; v < 4; ++v) H[nt][pt][v] *= decay;
#pragma unroll
        for (int k = 0; k < kQ; k += 32) {
            float wk[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) wk[e] = lds.w[k + 8 * g + e];
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt) {
                bf16x8 bw = lds8(&lds.Bt[nw0 + 16 * nt + c][k + 8 * g]);
#pragma unroll
                for (int e = 0; e < 8; ++e) bw[e] = static_cast<__bf16>(static_cast<float>(bw[e]) * wk[e]);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
                    H[nt][pt] = mfma16(bw, lds8(&lds.Xt[16 * pt + c][k + 8 * g]), H[nt][pt]);
            }
        }
        __syncthreads();
    }

    if (a.hL != nullptr) {
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int n = nw0 + 16 * nt + 4 * g + v, p = 16 * pt + c;
                    a.hL[((bb * a.nheads + hd) * kP + p) * N + n] = H[nt][pt][v];
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
