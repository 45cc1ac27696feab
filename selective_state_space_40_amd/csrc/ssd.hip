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
// the same permutation) and M never goes through LDS. C is read only by the
// wave that owns the token, so each lane keeps its token's C row in
// registers in operand layout. The chunk's x and B are staged once in LDS
// as they lie in memory (token rows, padded); the products that
// contract over tokens take them through the LDS transpose read, and the
// next chunk's inputs (x, B, C, z and the steps) are loaded into registers
// while this one is computed; nothing in the chunk waits on global memory
// until the next chunk is staged. bf16 I/O, head size 64, N = 64 or 128,
// Q = 64.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace mamba {
namespace {

constexpr int kQ = 64;   // tokens per chunk
constexpr int kP = 64;   // channels per head
constexpr int kSsdThreads = 256;
// Cache policy of the y stores: non-temporal (y is written once and not
// read back here).
constexpr int kStoreNt = 2;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

template <int N>
struct SsdLds {
    static constexpr int kRowN = N + 8;   // padded row of N bf16
    // padded row of 64 bf16 (x): 32 bytes of padding measured 210.5 us
    // against 212.3 us with 16 and 210.7 us with 48 on the Mamba-2 layer
    static constexpr int kRowQ = kQ + 16;
    __bf16 B[kQ][kRowN];     // B rows (j, n)
    __bf16 X[kQ][kRowQ];     // x rows (j, p)
    __bf16 H[kP][kRowN];     // the state entering the chunk (p, n)
    // Per-token values of a chunk, double-buffered by chunk parity: wave 0
    // forms those of the next chunk at the end of the current one.
    struct Steps {
        alignas(16) float dt[kQ];  // the step as used
        float S[kQ];               // log2 of the decay from chunk start through token j
        float w[kQ];               // exp(S_last - S_j) dt_j: weight of token j in the state update
    } st[2];
    alignas(16) float D[kP];   // the skip weights of the head's channels
    float Y[4][16][kP + 4];    // per wave: its 16 tokens' outputs before the gate (i, p)
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const __bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// Operands that contract over tokens read a token-major LDS tile T (rows of
// RS bf16) through the LDS transpose read (ds_read_b64_tr_b16). Within each
// group of 16 lanes, lane r receives element (r mod 4) of the 8 bytes that
// lane 4e + r/4 of its group addresses, as its element e. So when lane s of
// the group addresses row R + s/4, columns C + 4 (s mod 4) .. + 3, lane r
// receives T[R + e][C + r] for e = 0..3: four consecutive K values of column
// C + r, as an MFMA operand takes them. Lane (c, g) of the operand gets
// T[r0 + e][c0 + c] as its K values 0..3 and T[r1 + e][c0 + c] as 4..7; r0
// and r1 may differ per group g.
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 lds_tr4(const __bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const_cast<__bf16*>(p)));
}

template <int RS>
__device__ __forceinline__ bf16x8 lds_tr8(const __bf16* T, int r0, int r1, int c0) {
    const int s = threadIdx.x & 15;
    const int off = (s >> 2) * RS + c0 + 4 * (s & 3);
    const s16x4 a = lds_tr4(T + r0 * RS + off);
    const s16x4 b = lds_tr4(T + r1 * RS + off);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// How the chunk's inputs are spread over the threads. 64 threads each
// load an 8 x 8 block (8 tokens, 8 channels) of x, N threads (N / 8
// blocks per 8 tokens) an 8 x 8 block of B; every lane loads the raw step
// of token `lane` (wave 0 forms the steps from it). Every lane loads the C row of its own token i as the
// products read it (8 values of n at 8 g + 32 k for k < N / 32), and the gate
// z and input x of 8 channels of two of its wave's tokens in row order (see
// the output step).
constexpr int kXWave = 3;  // the wave that stages x

template <int N>
struct Layout {
    static constexpr int kXBlocks = (kQ / 8) * (kP / 8);
    static constexpr int kBBlocks = (kQ / 8) * (N / 8);
    static constexpr int kCk = N / 32;   // K steps of 32 over n
};

// Buffer resource over `bytes` bytes from p (raw addressing, gfx9 word 3):
// a load whose offset lies at or past the end returns zeros, so the tokens
// of a ragged last chunk need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}


// The loads of chunk [t0, t0 + cnt) of row bb, head hd, in three groups
// issued at different points of the previous chunk: each group goes into
// the registers that held the previous chunk's values right after their last
// use, so no registers are copied between chunks. Every resource starts at
// the chunk's first token and ends after its last valid one; lane offsets
// are the same for every chunk. Offsets fit 31 bits since the library caps
// nheads at 2^16 (64 rows of 2^22 channels).
struct ChunkPos {
    int64_t row0;   // bb * seqlen + t0
    int cnt;        // valid tokens
};

// x and B blocks and the step, consumed when the chunk is staged. One load
// sequence for every wave (a branch per tensor would merge the loaded
// registers through copies that wait for the loads): wave 3, which has the
// most causal work but nothing else before the staging barrier, loads x
// blocks, waves 1 (and 2 for N = 128) B blocks, any other wave an empty
// range; wave 0 forms the steps of the chunk ahead.
template <int N>
__device__ __forceinline__ void fetch_tiles(const SsdArgs& a, int64_t hd, ChunkPos c,
                                            uint4 (&blk)[8], uint32_t& dt) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int dim = static_cast<int>(a.nheads) * kP;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const bool isx = wv == kXWave;
    const bool isb = wv >= 1 && wv < kXWave && (wv - 1) * kWave < Layout<N>::kBBlocks;
    const __amdgpu_buffer_rsrc_t rx = chunk_rsrc(
        static_cast<const uint16_t*>(a.x) + c.row0 * dim + hd * kP, ((c.cnt - 1) * dim + kP) * 2);
    const __amdgpu_buffer_rsrc_t rb =
        chunk_rsrc(static_cast<const uint16_t*>(a.B) + c.row0 * N, isb ? c.cnt * N * 2 : 0);
    const int xe = tid - kXWave * kWave, e = tid - kWave;
    const int off = isx ? ((xe / (kP / 8)) * 8 * dim + 8 * (xe % (kP / 8))) * 2
                        : ((e / (N / 8)) * 8 * N + 8 * (e % (N / 8))) * 2;
    const int step = isx ? dim * 2 : N * 2;
    const __amdgpu_buffer_rsrc_t rblk = isx ? rx : rb;
#pragma unroll
    for (int r = 0; r < 8; ++r) blk[r] = ld128(rblk, off + r * step);
    const int nh = static_cast<int>(a.nheads);
    const __amdgpu_buffer_rsrc_t rdt = chunk_rsrc(static_cast<const uint16_t*>(a.dt) + c.row0 * nh + hd,
                                                  ((c.cnt - 1) * nh + 1) * 2);
    dt = static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(rdt, lane * nh * 2, 0, 0));
}

// This lane's C row as the products read it; last used by the H C^T product.
template <int N>
__device__ __forceinline__ void fetch_c(const SsdArgs& a, ChunkPos c, bf16x8 (&cop)[Layout<N>::kCk]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int i = 16 * (threadIdx.x / kWave) + (lane & 15), g = lane >> 4;
    const __amdgpu_buffer_rsrc_t rc =
        chunk_rsrc(static_cast<const uint16_t*>(a.C) + c.row0 * N, c.cnt * N * 2);
#pragma unroll
    for (int k = 0; k < Layout<N>::kCk; ++k)
        cop[k] = __builtin_bit_cast(bf16x8, ld128(rc, (i * N + 8 * g + 32 * k) * 2));
}

// The gate and input rows of the output step (rows 16 w + (lane / 8) + 8 h,
// channels 8 (lane % 8) .. + 8); last used by the output step.
template <bool HAS_D, bool HAS_Z>
__device__ __forceinline__ void fetch_out(const SsdArgs& a, int64_t hd, ChunkPos c, uint4 (&zc)[2],
                                          uint4 (&xc)[2]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int dim = static_cast<int>(a.nheads) * kP;
    const int span = ((c.cnt - 1) * dim + kP) * 2;
    const int orow = 16 * (threadIdx.x / kWave) + (lane >> 3), ocol = 8 * (lane & 7);
    if constexpr (HAS_Z) {
        const __amdgpu_buffer_rsrc_t rz =
            chunk_rsrc(static_cast<const uint16_t*>(a.z) + c.row0 * dim + hd * kP, span);
#pragma unroll
        for (int h = 0; h < 2; ++h) zc[h] = ld128(rz, ((orow + 8 * h) * dim + ocol) * 2);
    }
    if constexpr (HAS_D) {
        const __amdgpu_buffer_rsrc_t rx =
            chunk_rsrc(static_cast<const uint16_t*>(a.x) + c.row0 * dim + hd * kP, span);
#pragma unroll
        for (int h = 0; h < 2; ++h) xc[h] = ld128(rx, ((orow + 8 * h) * dim + ocol) * 2);
    }
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2,
// 4 and 8 within rows of 16 lanes, then the row totals are carried with the
// row broadcasts of lanes 15 and 31.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}

__device__ __forceinline__ float wave_prefix_sum(float v) {
    v = dpp_add<0x111, 0xf>(v);   // row_shr:1
    v = dpp_add<0x112, 0xf>(v);   // row_shr:2
    v = dpp_add<0x114, 0xf>(v);   // row_shr:4
    v = dpp_add<0x118, 0xf>(v);   // row_shr:8
    v = dpp_add<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}

template <int N, bool SP, bool HAS_D, bool HAS_Z>
__global__ __launch_bounds__(kSsdThreads) __attribute__((amdgpu_waves_per_eu(2)))
void ssd_fwd_kernel(SsdArgs a) {
    constexpr int NW = N / 4;        // state rows n per wave
    constexpr int NTN = NW / 16;     // 16-row blocks of them
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
    const int tb = w;                // this wave's block of 16 tokens
    const int i = 16 * tb + c;       // this lane's token of the chunk (as output column)

    // state H^T: block (nt, pt) holds rows n = nw0 + 16 nt + 4 g + v, column p = 16 pt + c
    const int nw0 = NW * w;
    if (tid < kP) lds.D[tid] = HAS_D ? a.D[hd * kP + tid] : 0.0f;
    // the 4 values of a lane's block are 4 consecutive states of one channel:
    // one 16-byte load (and, at the end, store) each
    f32x4 H[NTN][4];
#pragma unroll
    for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const int n = nw0 + 16 * nt + 4 * g, p = 16 * pt + c;
            H[nt][pt] = a.h0 != nullptr
                            ? *reinterpret_cast<const f32x4*>(&a.h0[((bb * a.nheads + hd) * kP + p) * N + n])
                            : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }

    const int64_t nchunks = (L + kQ - 1) / kQ;
    // the chunk whose loads a step issues: the next one, the last one
    // loading itself again (unused) so that every iteration issues the same
    // loads and the waits before each use stay exact
    auto pos = [&](int64_t k) {
        k = min(k, nchunks - 1);
        return ChunkPos{bb * L + k * kQ, static_cast<int>(min<int64_t>(kQ, L - k * kQ))};
    };
    uint4 blk[8], zc[2], xc[2];
    uint32_t dtr;
    bf16x8 cop[Layout<N>::kCk];
    // Wave 0: the steps of a chunk of cnt_k tokens from their raw values in
    // dtr, their running sum (a DPP prefix sum) and the token weights.
    auto form_steps = [&](typename SsdLds<N>::Steps& o, int cnt_k) {
        const float v = raw_to_f32<kIoBF16>(dtr) + bias;
        const float dtv = lane < cnt_k ? (SP ? softplus_f32(v) : v) : 0.0f;
        const float s = wave_prefix_sum(dtv) * alog2;
        const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), kWave - 1));
        o.dt[lane] = dtv;
        o.S[lane] = s;
        o.w[lane] = fast_exp2(last - s) * dtv;
    };
    fetch_tiles<N>(a, hd, pos(0), blk, dtr);
    fetch_c<N>(a, pos(0), cop);
    fetch_out<HAS_D, HAS_Z>(a, hd, pos(0), zc, xc);
    if (w == 0) form_steps(lds.st[0], pos(0).cnt);
    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t t0 = ch * kQ;
        const int cnt = static_cast<int>(min<int64_t>(kQ, L - t0));

        // (1) stage the chunk: x and B rows as they are and the state
        // entering the chunk as bf16 (p, n); its steps were formed at the end
        // of the chunk before
        const typename SsdLds<N>::Steps& sp = lds.st[ch & 1];
        if (w == kXWave) {
            const int xe = tid - kXWave * kWave;
            const int jb = xe / (kP / 8), pb = xe % (kP / 8);
#pragma unroll
            for (int f = 0; f < 8; ++f) *reinterpret_cast<uint4*>(&lds.X[8 * jb + f][8 * pb]) = blk[f];
        } else if (w >= 1 && tid - kWave < Layout<N>::kBBlocks) {
            const int e = tid - kWave;
            const int jb = e / (N / 8), nb = e % (N / 8);
#pragma unroll
            for (int f = 0; f < 8; ++f) *reinterpret_cast<uint4*>(&lds.B[8 * jb + f][8 * nb]) = blk[f];
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

        // the next chunk's tiles and steps go out now and land during this one
        fetch_tiles<N>(a, hd, pos(ch + 1), blk, dtr);
        const float s_last = sp.S[kQ - 1];

        // (3) M^T for this wave's tokens: blocks jt = 0 .. w of G^T = B C^T
        f32x4 Mt[4];
        const float si = sp.S[i];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            Mt[jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (jt <= tb) {
#pragma unroll
                for (int k = 0; k < N; k += 32)
                    Mt[jt] = mfma16(lds8(&lds.B[16 * jt + c][k + 8 * g]), cop[k / 32], Mt[jt]);
                // token j = 16 jt + 4 g + v; above the diagonal (j > i) the
                // factor may overflow and is discarded by the select
                const f32x4 sj = *reinterpret_cast<const f32x4*>(&sp.S[16 * jt + 4 * g]);
                const f32x4 dj = *reinterpret_cast<const f32x4*>(&sp.dt[16 * jt + 4 * g]);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float e = fast_exp2(si - sj[v]) * dj[v];
                    Mt[jt][v] = (jt < tb || 4 * g + v <= c) ? Mt[jt][v] * e : 0.0f;
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
            if (2 * s2 <= tb) {
                // K = 32 tokens j: j = 32 s2 + 4 g + e (e < 4) and 32 s2 + 16 + 4 g + (e - 4)
                bf16x8 mb;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    mb[e] = static_cast<__bf16>(Mt[2 * s2][e]);
                    mb[e + 4] = static_cast<__bf16>(Mt[2 * s2 + 1][e]);
                }
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
                    Yd[pt] = mfma16(lds_tr8<SsdLds<N>::kRowQ>(&lds.X[0][0], 32 * s2 + 4 * g,
                                                              32 * s2 + 16 + 4 * g, 16 * pt),
                                    mb, Yd[pt]);
            }
        }
#pragma unroll
        for (int k = 0; k < N; k += 32) {
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
                Yo[pt] = mfma16(lds8(&lds.H[16 * pt + c][k + 8 * g]), cop[k / 32], Yo[pt]);
        }
        // this chunk's C is no longer needed: the next chunk's goes out
        fetch_c<N>(a, pos(ch + 1), cop);
        // (5) output: the wave's 16 x 64 block leaves the accumulators through
        // LDS so that the gate and input are read, and y written, as whole
        // rows (16 bytes per lane, 8 lanes per row); rows past the sequence
        // end fall outside the chunk's buffer range and are not stored.
        {
            const float eo = fast_exp2(si);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                f32x4 o;
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = fmaf(eo, Yo[pt][v], Yd[pt][v]);
                *reinterpret_cast<f32x4*>(&lds.Y[w][c][16 * pt + 4 * g]) = o;
            }
            // lanes of this wave read what other lanes of it wrote
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int orow = lane >> 3, ocol = 8 * (lane & 7);
            const __amdgpu_buffer_rsrc_t ry =
                chunk_rsrc(static_cast<uint16_t*>(a.y) + (bb * L + t0) * dim + hd * kP,
                           ((cnt - 1) * static_cast<int>(dim) + kP) * 2);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = orow + 8 * h;
                const f32x4 y0 = *reinterpret_cast<const f32x4*>(&lds.Y[w][r][ocol]);
                const f32x4 y1 = *reinterpret_cast<const f32x4*>(&lds.Y[w][r][ocol + 4]);
                float out[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
                if constexpr (HAS_D) {
                    const f32x4 d0 = *reinterpret_cast<const f32x4*>(&lds.D[ocol]);
                    const f32x4 d1 = *reinterpret_cast<const f32x4*>(&lds.D[ocol + 4]);
                    const uint32_t xw[4] = {xc[h].x, xc[h].y, xc[h].z, xc[h].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        out[2 * e] = fmaf(e < 2 ? d0[2 * e] : d1[2 * e - 4], __uint_as_float(xw[e] << 16), out[2 * e]);
                        out[2 * e + 1] = fmaf(e < 2 ? d0[2 * e + 1] : d1[2 * e - 3],
                                              __uint_as_float(xw[e] & 0xffff0000u), out[2 * e + 1]);
                    }
                }
                if constexpr (HAS_Z) {
                    const uint32_t zw[4] = {zc[h].x, zc[h].y, zc[h].z, zc[h].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        out[2 * e] *= silu(__uint_as_float(zw[e] << 16));
                        out[2 * e + 1] *= silu(__uint_as_float(zw[e] & 0xffff0000u));
                    }
                }
                uint32_t ow[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ow[e] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(out[2 * e]))) |
                            (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(out[2 * e + 1]))) << 16);
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(__attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t,
                                       make_uint4(ow[0], ow[1], ow[2], ow[3])),
                    ry, ((16 * tb + r) * static_cast<int>(dim) + ocol) * 2, 0, kStoreNt);
            }
        }
        // nor this chunk's gate and input
        fetch_out<HAS_D, HAS_Z>(a, hd, pos(ch + 1), zc, xc);

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
            for (int e = 0; e < 8; ++e) wk[e] = sp.w[k + 8 * g + e];
            bf16x8 xo[4];
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
                xo[pt] = lds_tr8<SsdLds<N>::kRowQ>(&lds.X[0][0], k + 8 * g, k + 8 * g + 4, 16 * pt);
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt) {
                bf16x8 bw = lds_tr8<SsdLds<N>::kRowN>(&lds.B[0][0], k + 8 * g, k + 8 * g + 4,
                                                      nw0 + 16 * nt);
#pragma unroll
                for (int e = 0; e < 8; ++e) bw[e] = static_cast<__bf16>(static_cast<float>(bw[e]) * wk[e]);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) H[nt][pt] = mfma16(bw, xo[pt], H[nt][pt]);
            }
        }
        // the next chunk's steps, by the wave with the least causal work
        // (its raw steps were loaded after this chunk was staged; the buffer
        // was last read in the chunk before this one)
        if (w == 0) form_steps(lds.st[(ch + 1) & 1], pos(ch + 1).cnt);
        __syncthreads();
    }

    if (a.hL != nullptr) {
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int n = nw0 + 16 * nt + 4 * g, p = 16 * pt + c;
                *reinterpret_cast<f32x4*>(&a.hL[((bb * a.nheads + hd) * kP + p) * N + n]) = H[nt][pt];
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
