// HIP kernels of the selective state-space scan for gfx950 (CDNA4).
//
// The recurrence (page "Mamba and State Space Models", world.lapla.si,
// sections "A State of Fixed Size" and "Chosen by the Token"), per batch row
// b, channel d and state n:
//     Abar = exp(delta*A[d,n]),  h[n] <- Abar*h[n] + delta*B[n]*x,
//     y = (sum_n C[n]*h[n] + D[d]*x) * silu(z).
//
// Work mapping. The scan is elementwise in (b, d) and sequential in t, and it
// is no dense contraction, so it runs on the vector ALUs, not the matrix
// cores. One lane owns one channel d of one batch row b for one chunk of
// tokens; its N states, its N decay rates A[d,:]*log2(e) and its running
// readout stay in VGPRs for the whole chunk, so the N-times-larger expanded
// state never leaves the register file (section "A Scan on the Chip": only
// inputs and outputs touch memory). A wave covers 64 consecutive channels,
// so every x/delta/z load and y store of a token is one contiguous 128-byte
// (bf16) or 256-byte (fp32) access. B[b,t,:] and C[b,t,:] are the same for
// all channels of a wave, so they are fetched with scalar loads into SGPRs,
// converted on the scalar unit and used straight from there by the vector
// FMAs: no LDS round trip and no VGPRs for them.
//
// x, delta and z are fetched one register tile of kTokenTile tokens ahead of
// the tokens being computed, so the HBM latency of a tile overlaps the
// arithmetic of the previous one.
//
// Long sequences are cut into chunks that run in parallel. Pass 1 runs each
// chunk from a zero state (chunk 0 from h0) and keeps only its end state and
// its decay product P = exp(A * sum(delta)). The carry pass folds the pairs
// in order with the associative combine (P_a, h_a) . (P_b, h_b) =
// (P_a*P_b, P_b*h_a + h_b) to get the true state entering every chunk, and
// pass 2 reruns each chunk from that state and writes y (the "parallel scan"
// of section "A Scan on the Chip"). P is formed from a chunk-local sum of
// delta, never from differences of long prefix sums.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace mamba {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int TT = kTokenTile;

// ---------------------------------------------------------------------------
// I/O element access. Raw values are kept as 32-bit integers until use so a
// prefetched tile is not forced to wait for its loads early.
template <int IO>
__device__ __forceinline__ uint32_t load_raw(const void* __restrict__ p, int64_t i) {
    if constexpr (IO == kIoF32) {
        return static_cast<const uint32_t*>(p)[i];
    } else {
        return static_cast<const uint16_t*>(p)[i];
    }
}

template <int IO>
__device__ __forceinline__ float raw_to_f32(uint32_t r) {
    if constexpr (IO == kIoF32) {
        return __uint_as_float(r);
    } else {
        return __uint_as_float(r << 16);  // bf16 -> fp32 is exact
    }
}

template <int IO>
__device__ __forceinline__ void store_io(void* __restrict__ p, int64_t i, float v) {
    if constexpr (IO == kIoF32) {
        static_cast<float*>(p)[i] = v;
    } else {
        static_cast<__bf16*>(p)[i] = static_cast<__bf16>(v);  // round to nearest even
    }
}

typedef __attribute__((address_space(4))) uint32_t kconst_u32;

// One row of N B- or C-values at element offset `row` (wave-uniform): with
// bf16 and even N the row is dword aligned and read as N/2 dwords, which the
// compiler turns into scalar loads; the two halves of a dword are widened on
// the scalar unit.
template <int N, int IO>
__device__ __forceinline__ void load_row(const void* __restrict__ p, int64_t row, float (&out)[N]) {
    if constexpr (IO == kIoBF16 && (N % 2 == 0)) {
        // B and C are never written while a scan runs: reading them through
        // the constant address space lets the compiler use scalar loads even
        // though the kernel also stores through buffer resources.
        const kconst_u32* q = (const kconst_u32*)(p) + row / 2;
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const uint32_t w = q[i];
            out[2 * i] = __uint_as_float(w << 16);
            out[2 * i + 1] = __uint_as_float(w & 0xffff0000u);
        }
    } else if constexpr (IO == kIoF32) {
        const kconst_u32* q = (const kconst_u32*)(p) + row;
#pragma unroll
        for (int n = 0; n < N; ++n) out[n] = __uint_as_float(q[n]);
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) out[n] = raw_to_f32<IO>(load_raw<IO>(p, row + n));
    }
}

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float fast_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// silu(z) = z / (1 + exp(-z))
__device__ __forceinline__ float silu(float z) {
    return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e));
}

// ---------------------------------------------------------------------------
// Per-wave addressing of one chunk. x, delta, z and y of the chunk are read
// and written through buffer resources whose base is the chunk's first token
// at the wave's first channel: token j of a lane is at byte offset
// j * row_bytes (a scalar offset, advanced on the scalar unit) plus the
// lane's fixed 32-bit channel offset (one VGPR for the whole chunk), so no
// vector ALU work goes into addresses. The resource's record count is the
// chunk's byte extent, which the plan keeps below 2^32.
struct ChunkIo {
    __amdgpu_buffer_rsrc_t x, delta, z, y;
    uint32_t row_bytes;   // bytes between consecutive tokens of one channel
    uint32_t lane_bytes;  // byte offset of this lane's channel within a token row
};

// Raw buffer resource word 3 for gfx9-family parts (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                             kRsrcWord3);
}

template <int IO>
__device__ __forceinline__ uint32_t buf_load(__amdgpu_buffer_rsrc_t r, uint32_t lane_bytes,
                                             uint32_t row_off) {
    if constexpr (IO == kIoF32) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(lane_bytes),
                                                    static_cast<int>(row_off), 0);
    } else {
        return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(lane_bytes),
                                                    static_cast<int>(row_off), 0);
    }
}

template <int IO>
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t lane_bytes,
                                          uint32_t row_off, float v) {
    if constexpr (IO == kIoF32) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(lane_bytes),
                                              static_cast<int>(row_off), 0);
    } else {
        const __bf16 hv = static_cast<__bf16>(v);  // round to nearest even
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, hv), r,
                                              static_cast<int>(lane_bytes),
                                              static_cast<int>(row_off), 0);
    }
}

// One token of the recurrence for one lane. Bt/Ct point at B[b,t,0] and
// C[b,t,0] (wave-uniform).
template <int N, int IO, bool WRITE_Y, bool HAS_D, bool HAS_Z>
__device__ __forceinline__ void scan_token(const ChunkIo& io, const void* Bt, const void* Ct,
                                           uint32_t row_off, uint32_t xr, uint32_t dr,
                                           uint32_t zr, const float (&A2)[N], float (&h)[N],
                                           float dskip, float& dsum) {
    const float dt = raw_to_f32<IO>(dr);
    const float u = raw_to_f32<IO>(xr);
    float Bv[N];
    load_row<N, IO>(Bt, 0, Bv);
    const float du = dt * u;
    if constexpr (WRITE_Y) {
        float Cv[N];
        load_row<N, IO>(Ct, 0, Cv);
        float acc = HAS_D ? dskip * u : 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float e = fast_exp2(dt * A2[n]);
            h[n] = fmaf(e, h[n], du * Bv[n]);
            acc = fmaf(Cv[n], h[n], acc);
        }
        if constexpr (HAS_Z) acc *= silu(raw_to_f32<IO>(zr));
        // Lanes past the last channel were clamped onto channel dim-1 and
        // computed its value bit for bit, so they store the same bits to the
        // same address; the store needs no lane mask and no branch.
        buf_store<IO>(io.y, io.lane_bytes, row_off, acc);
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float e = fast_exp2(dt * A2[n]);
            h[n] = fmaf(e, h[n], du * Bv[n]);
        }
        dsum += dt;
    }
}

template <int IO, bool LOAD_Z>
__device__ __forceinline__ void fetch_tile(const ChunkIo& io, int tile, uint32_t (&xr)[TT],
                                           uint32_t (&dr)[TT], uint32_t (&zr)[TT]) {
#pragma unroll
    for (int j = 0; j < TT; ++j) {
        const uint32_t off = static_cast<uint32_t>(tile * TT + j) * io.row_bytes;
        xr[j] = buf_load<IO>(io.x, io.lane_bytes, off);
        dr[j] = buf_load<IO>(io.delta, io.lane_bytes, off);
        zr[j] = LOAD_Z ? buf_load<IO>(io.z, io.lane_bytes, off) : 0u;
    }
}

template <int N, int IO, bool WRITE_Y, bool HAS_D, bool HAS_Z>
__device__ __forceinline__ void compute_tile(const ChunkIo& io, const char* Bc, const char* Cc,
                                             int tile, const uint32_t (&xr)[TT],
                                             const uint32_t (&dr)[TT], const uint32_t (&zr)[TT],
                                             const float (&A2)[N], float (&h)[N], float dskip,
                                             float& dsum) {
    constexpr int64_t kRowBytes = N * (IO == kIoF32 ? 4 : 2);
#pragma unroll
    for (int j = 0; j < TT; ++j) {
        const int tok = tile * TT + j;
        scan_token<N, IO, WRITE_Y, HAS_D, HAS_Z>(io, Bc + tok * kRowBytes, Cc + tok * kRowBytes,
                                                 static_cast<uint32_t>(tok) * io.row_bytes, xr[j],
                                                 dr[j], zr[j], A2, h, dskip, dsum);
    }
}

// All `ntok` tokens of one lane's chunk. Bc/Cc point at B[b,t0,0] and
// C[b,t0,0]. Two register tiles alternate: while one tile of tokens is
// computed the next one is already in flight, and the tiles swap roles
// without register copies.
template <int N, int IO, bool WRITE_Y, bool HAS_D, bool HAS_Z>
__device__ __forceinline__ void scan_chunk(const ChunkIo& io, const char* Bc, const char* Cc,
                                           int ntok, const float (&A2)[N], float (&h)[N],
                                           float dskip, float& dsum) {
    constexpr bool LOAD_Z = WRITE_Y && HAS_Z;
    constexpr int64_t kRowBytes = N * (IO == kIoF32 ? 4 : 2);
    const int ntiles = ntok / TT;
    if (ntiles > 0) {
        // The fetch is unconditional (past the last tile it re-reads the last
        // tile, whose values go unused) so every path into a compute step has
        // the same loads in flight and the waits before it stay exact.
        uint32_t xa[TT], da[TT], za[TT], xb[TT], db[TT], zb[TT];
        fetch_tile<IO, LOAD_Z>(io, 0, xa, da, za);
        int i = 0;
        while (true) {
            fetch_tile<IO, LOAD_Z>(io, min(i + 1, ntiles - 1), xb, db, zb);
            compute_tile<N, IO, WRITE_Y, HAS_D, HAS_Z>(io, Bc, Cc, i, xa, da, za, A2, h, dskip, dsum);
            if (++i == ntiles) break;
            fetch_tile<IO, LOAD_Z>(io, min(i + 1, ntiles - 1), xa, da, za);
            compute_tile<N, IO, WRITE_Y, HAS_D, HAS_Z>(io, Bc, Cc, i, xb, db, zb, A2, h, dskip, dsum);
            if (++i == ntiles) break;
        }
    }
    for (int tok = ntiles * TT; tok < ntok; ++tok) {  // ragged tail, fewer than TT tokens
        const uint32_t off = static_cast<uint32_t>(tok) * io.row_bytes;
        const uint32_t zr = LOAD_Z ? buf_load<IO>(io.z, io.lane_bytes, off) : 0u;
        scan_token<N, IO, WRITE_Y, HAS_D, HAS_Z>(
            io, Bc + tok * kRowBytes, Cc + tok * kRowBytes, off,
            buf_load<IO>(io.x, io.lane_bytes, off), buf_load<IO>(io.delta, io.lane_bytes, off), zr,
            A2, h, dskip, dsum);
    }
}

struct ChunkGrid {
    int64_t nblk_d;     // channel groups per batch row
    int64_t nchunks;    // chunks per sequence
    int64_t chunk_len;  // tokens per chunk
};

__device__ __forceinline__ void decode_block(const ChunkGrid& g, int64_t blk, int64_t& dblk,
                                             int64_t& k, int64_t& b) {
    dblk = blk % g.nblk_d;
    const int64_t r = blk / g.nblk_d;
    k = r % g.nchunks;
    b = r / g.nchunks;
}

// Workspace pointers: three [nchunks][batch][dim][N] fp32 arrays.
struct Carry {
    float* start;  // state entering chunk k (k = 0: a copy of h0)
    float* end;    // end state of chunk k from a zero start (k = 0: from h0)
    float* decay;  // exp(A * sum of delta over chunk k)
};

// Pass 1: per-chunk summaries (end state, decay product), all chunks but the
// last. Chunk 0 starts from h0, so its end state is already exact.
template <int N, int IO>
__global__ __launch_bounds__(kWave) void chunk_summary_kernel(ScanArgs a, ChunkGrid g, Carry c) {
    int64_t dblk, k, b;
    decode_block(g, blockIdx.x, dblk, k, b);
    // lanes past the last channel work on channel dim-1 (see scan_token)
    const int64_t d0 = dblk * kWave;
    const int64_t d = min(d0 + static_cast<int64_t>(threadIdx.x), a.dim - 1);
    const int64_t t0 = k * g.chunk_len;
    const int64_t t1 = min(a.seqlen, t0 + g.chunk_len);
    const int ntok = static_cast<int>(t1 - t0);
    constexpr int64_t esz = IO == kIoF32 ? 4 : 2;
    const int64_t first = (b * a.seqlen + t0) * a.dim + d0;  // element (b, t0, d0)
    // bytes from (b, t0, d0) to the end of (b, t1-1, dim-1); below 2^32 by the plan
    const uint32_t extent = static_cast<uint32_t>(((t1 - t0) * a.dim - d0) * esz);
    ChunkIo io;
    io.row_bytes = static_cast<uint32_t>(a.dim * esz);
    io.lane_bytes = static_cast<uint32_t>((d - d0) * esz);
    io.x = make_rsrc(static_cast<const char*>(a.x) + first * esz, extent);
    io.delta = make_rsrc(static_cast<const char*>(a.delta) + first * esz, extent);
    io.z = make_rsrc(a.z != nullptr ? static_cast<const char*>(a.z) + first * esz : nullptr, extent);
    io.y = make_rsrc(static_cast<const char*>(a.y) + first * esz, extent);
    const char* Bc = static_cast<const char*>(a.B) + (b * a.seqlen + t0) * N * esz;
    const char* Cc = static_cast<const char*>(a.C) + (b * a.seqlen + t0) * N * esz;

    float A2[N], h[N];
    const int64_t srow = ((k * a.batch + b) * a.dim + d) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.A[d * N + n] * kLog2e;
        h[n] = (k == 0 && a.h0 != nullptr) ? a.h0[(b * a.dim + d) * N + n] : 0.0f;
    }
    if (k == 0) {
#pragma unroll
        for (int n = 0; n < N; ++n) c.start[srow + n] = h[n];
    }
    float dsum = 0.0f;
    scan_chunk<N, IO, false, false, false>(io, Bc, Cc, ntok, A2, h, 0.0f, dsum);
#pragma unroll
    for (int n = 0; n < N; ++n) {
        c.end[srow + n] = h[n];
        c.decay[srow + n] = fast_exp2(A2[n] * dsum);
    }
}

// Carry pass: one thread per (b, d, n) column folds the chunk summaries in
// order and writes the state entering chunks 1 .. nchunks-1.
__global__ __launch_bounds__(256) void chunk_carry_kernel(int64_t columns, int64_t nchunks,
                                                          Carry c) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t col = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; col < columns;
         col += stride) {
        float H = c.end[col];  // exact end state of chunk 0
        for (int64_t k = 1; k < nchunks; ++k) {
            c.start[k * columns + col] = H;
            if (k + 1 < nchunks) H = fmaf(c.decay[k * columns + col], H, c.end[k * columns + col]);
        }
    }
}

// Pass 2 (or the only pass when nchunks == 1): scan each chunk from its true
// entering state and write y; the last chunk writes hL.
template <int N, int IO, bool HAS_D, bool HAS_Z>
__global__ __launch_bounds__(kWave) void chunk_output_kernel(ScanArgs a, ChunkGrid g, Carry c) {
    int64_t dblk, k, b;
    decode_block(g, blockIdx.x, dblk, k, b);
    // lanes past the last channel work on channel dim-1 (see scan_token)
    const int64_t d0 = dblk * kWave;
    const int64_t d = min(d0 + static_cast<int64_t>(threadIdx.x), a.dim - 1);
    const int64_t t0 = k * g.chunk_len;
    const int64_t t1 = min(a.seqlen, t0 + g.chunk_len);
    const int ntok = static_cast<int>(t1 - t0);
    constexpr int64_t esz = IO == kIoF32 ? 4 : 2;
    const int64_t first = (b * a.seqlen + t0) * a.dim + d0;  // element (b, t0, d0)
    // bytes from (b, t0, d0) to the end of (b, t1-1, dim-1); below 2^32 by the plan
    const uint32_t extent = static_cast<uint32_t>(((t1 - t0) * a.dim - d0) * esz);
    ChunkIo io;
    io.row_bytes = static_cast<uint32_t>(a.dim * esz);
    io.lane_bytes = static_cast<uint32_t>((d - d0) * esz);
    io.x = make_rsrc(static_cast<const char*>(a.x) + first * esz, extent);
    io.delta = make_rsrc(static_cast<const char*>(a.delta) + first * esz, extent);
    io.z = make_rsrc(a.z != nullptr ? static_cast<const char*>(a.z) + first * esz : nullptr, extent);
    io.y = make_rsrc(static_cast<const char*>(a.y) + first * esz, extent);
    const char* Bc = static_cast<const char*>(a.B) + (b * a.seqlen + t0) * N * esz;
    const char* Cc = static_cast<const char*>(a.C) + (b * a.seqlen + t0) * N * esz;

    float A2[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) A2[n] = a.A[d * N + n] * kLog2e;
    if (g.nchunks == 1) {
#pragma unroll
        for (int n = 0; n < N; ++n)
            h[n] = a.h0 != nullptr ? a.h0[(b * a.dim + d) * N + n] : 0.0f;
    } else {
        const int64_t srow = ((k * a.batch + b) * a.dim + d) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = c.start[srow + n];
    }
    const float dskip = HAS_D ? a.D[d] : 0.0f;
    float dsum = 0.0f;
    scan_chunk<N, IO, true, HAS_D, HAS_Z>(io, Bc, Cc, ntok, A2, h, dskip, dsum);
    if (k == g.nchunks - 1 && a.hL != nullptr) {
#pragma unroll
        for (int n = 0; n < N; ++n) a.hL[(b * a.dim + d) * N + n] = h[n];
    }
}

// seqlen == 0: hL = h0 (or zeros).
__global__ __launch_bounds__(256) void state_init_kernel(int64_t count, const float* h0,
                                                         float* hL) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
         i += stride)
        hL[i] = h0 != nullptr ? h0[i] : 0.0f;
}

// Grid for the grid-stride kernels above: enough 256-thread blocks to cover
// `count` items, capped well below the 32-bit grid limit.
inline int64_t stride_blocks(int64_t count) {
    const int64_t b = (count + 255) / 256;
    return b < (int64_t(1) << 20) ? (b > 0 ? b : 1) : (int64_t(1) << 20);
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
        const float4 h4 = *reinterpret_cast<const float4*>(hrow);
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
    const float dt = raw_to_f32<IO>(load_raw<IO>(a.delta, p));
    const float u = raw_to_f32<IO>(load_raw<IO>(a.x, p));
    const float du = dt * u;
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const float e = fast_exp2(dt * (Av[s] * kLog2e));
        hv[s] = fmaf(e, hv[s], du * Bv[s]);
        acc = fmaf(Cv[s], hv[s], acc);
    }
    acc = group_sum<G>(acc);
    if constexpr (HAS_D) acc = fmaf(a.D[d], u, acc);
    if constexpr (HAS_Z) acc *= silu(raw_to_f32<IO>(load_raw<IO>(a.z, p)));
    if (live) {
        if constexpr (S == 4) {
            *reinterpret_cast<float4*>(hrow) = make_float4(hv[0], hv[1], hv[2], hv[3]);
        } else {
#pragma unroll
            for (int s = 0; s < S; ++s) hrow[s] = hv[s];
        }
        if (part == 0) store_io<IO>(a.y, p, acc);
    }
}

// ---------------------------------------------------------------------------
// Host-side dispatch over the compile-time variants.
template <int N, int IO>
hipError_t launch_scan_n(const ScanArgs& a, const ScanPlan& plan, void* ws, hipStream_t s) {
    ChunkGrid g;
    g.nblk_d = (a.dim + kWave - 1) / kWave;
    g.nchunks = plan.nchunks;
    g.chunk_len = plan.chunk_len;
    Carry c{nullptr, nullptr, nullptr};
    const int64_t columns = a.batch * a.dim * N;
    if (plan.nchunks > 1) {
        float* base = static_cast<float*>(ws);
        c.start = base;
        c.end = base + plan.nchunks * columns;
        c.decay = base + 2 * plan.nchunks * columns;
        const int64_t blocks1 = g.nblk_d * (plan.nchunks - 1) * a.batch;
        // pass 1 covers chunks 0 .. nchunks-2; its grid uses nchunks-1 as the
        // chunk count so block indices map onto exactly those chunks
        ChunkGrid g1 = g;
        g1.nchunks = plan.nchunks - 1;
        hipLaunchKernelGGL((chunk_summary_kernel<N, IO>), dim3(blocks1), dim3(kWave), 0, s, a, g1,
                           c);
        // g1 indexes chunks like g (k * chunk_len), only fewer of them; the
        // workspace rows use the full nchunks stride through `columns`.
        hipLaunchKernelGGL(chunk_carry_kernel, dim3(stride_blocks(columns)), dim3(256), 0, s,
                           columns, plan.nchunks, c);
    }
    const int64_t blocks = g.nblk_d * plan.nchunks * a.batch;
    const bool has_d = a.D != nullptr, has_z = a.z != nullptr;
    if (has_d && has_z)
        hipLaunchKernelGGL((chunk_output_kernel<N, IO, true, true>), dim3(blocks), dim3(kWave), 0, s, a, g, c);
    else if (has_d)
        hipLaunchKernelGGL((chunk_output_kernel<N, IO, true, false>), dim3(blocks), dim3(kWave), 0, s, a, g, c);
    else if (has_z)
        hipLaunchKernelGGL((chunk_output_kernel<N, IO, false, true>), dim3(blocks), dim3(kWave), 0, s, a, g, c);
    else
        hipLaunchKernelGGL((chunk_output_kernel<N, IO, false, false>), dim3(blocks), dim3(kWave), 0, s, a, g, c);
    return hipGetLastError();
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
hipError_t dispatch_scan(const ScanArgs& a, const ScanPlan& p, void* ws, hipStream_t s) {
    switch (a.dstate) {
#define MAMBA_CASE(n) case n: return launch_scan_n<n, IO>(a, p, ws, s);
        MAMBA_CASE(1) MAMBA_CASE(2) MAMBA_CASE(3) MAMBA_CASE(4) MAMBA_CASE(5) MAMBA_CASE(6)
        MAMBA_CASE(7) MAMBA_CASE(8) MAMBA_CASE(9) MAMBA_CASE(10) MAMBA_CASE(11) MAMBA_CASE(12)
        MAMBA_CASE(13) MAMBA_CASE(14) MAMBA_CASE(15) MAMBA_CASE(16)
#undef MAMBA_CASE
        default: return hipErrorInvalidValue;
    }
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
    return a.io == kIoF32 ? dispatch_scan<kIoF32>(a, plan, workspace, stream)
                          : dispatch_scan<kIoBF16>(a, plan, workspace, stream);
}

hipError_t launch_state_update(const DecodeArgs& a, hipStream_t stream) {
    return a.io == kIoF32 ? dispatch_decode<kIoF32>(a, stream)
                          : dispatch_decode<kIoBF16>(a, stream);
}

}  // namespace mamba
