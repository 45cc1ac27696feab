// HIP kernels of the selective state-space scan for gfx950 (CDNA4).
//
// The recurrence (page "Mamba and State Space Models", world.lapla.si,
// sections "A State of Fixed Size" and "Chosen by the Token"), per batch row
// b, channel d and state n:
//     Abar = exp(delta*A[d,n]),  h[n] <- Abar*h[n] + delta*B[n]*x,
//     y = (sum_n C[n]*h[n] + D[d]*x) * silu(z).
// Delta may arrive raw: the kernels then add a per-channel bias and apply
// softplus as they convert each (channel, token) once, and every later use,
// the chunk sums of pass 1 included, sees the activated value.
//
// Work mapping. The scan is elementwise in (b, d) and sequential in t, and it
// is no dense contraction, so it runs on the vector ALUs, not the matrix
// cores. A workgroup covers 64 consecutive channels of one batch row over
// one chunk of tokens, one channel per lane; its S waves split the N states
// of each channel, so a lane keeps N/S states and N/S decay rates
// A[d,n]*log2(e) in VGPRs for the whole chunk and the N-times-larger expanded
// state never leaves the register file (section "A Scan on the Chip": only
// inputs and outputs touch memory). Every x/delta/z load and y store of a
// token is one contiguous 128-byte (bf16) or 256-byte (fp32) access of the
// wave. B[b,t,:] and C[b,t,:] are shared by all channels: the workgroup
// stages each tile's rows in LDS as fp32 and every wave reads its slice with
// broadcast LDS reads. The S partial readouts of a token are summed through
// LDS, and the epilogue (skip term, silu gate, bf16 rounding, store) is
// spread over the S waves.
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
//
// With long chunks the carry can instead be repaired where it matters. Pass
// 1 then runs every chunk once from a zero state (chunk 0 from h0) and
// writes y as well as the summary pair; the carry pass folds the pairs
// through the last chunk, which gives hL too. The true state of a chunk
// differs from its zero-start state by P_t (.) h_in, where P_t =
// exp(A * sum of delta since the chunk start) only shrinks along the chunk
// (delta > 0, A < 0), so pass 2 reruns each later chunk from its entering
// state only until P_t <= 2^-32 for every state of the workgroup, and the
// zero-start outputs stand from there on: what they leave out is below
// 2^-32 * sum_n |C[n] h_in[n]|, under the fp32 rounding of that readout.
// The stopping test is made on the data, so the cost depends on the decay;
// where the weight never falls (A >= 0, delta = 0, NaN) pass 2 reruns the
// whole chunk, as the two-pass form does.
//
// This header is the body of scan_variant.hip, which is compiled once per
// (I/O dtype, delta activation, dstate half) so the variants build in
// parallel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace mamba {
namespace {

// ---------------------------------------------------------------------------
// Per-wave addressing of one chunk. x, delta, z and y of the chunk are read
// and written through buffer resources whose base is the chunk's first token
// at the workgroup's first channel: token j of a lane is at byte offset
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

// ---------------------------------------------------------------------------
// Work mapping. A workgroup of S waves covers 64 consecutive channels of one
// batch row over one chunk of tokens, and its S waves split the N states of
// every channel: wave w owns states [w*N/S, (w+1)*N/S). Each wave therefore
// needs only its slice of B[b,t,:] and C[b,t,:], which is the same for all
// 64 lanes and lives in SGPRs, and keeps N/S states and N/S decay rates per
// lane. Splitting the states multiplies the waves of a launch by S without
// the extra summary pass a further split of the sequence would cost; the
// price is that the per-token conversions of x and delta are repeated in
// each of the S waves and that the readout is summed across waves.
//
// The readout of a register tile of TT tokens is summed through LDS: every
// wave writes its partial sums C.h over its states for the TT tokens, one
// barrier, and wave w then finalises the tokens j = w, w+S, ... of the tile
// (sum of the S partials in a fixed order, skip term, silu gate, rounding and
// store), so the epilogue work is spread evenly over the S waves. The LDS
// buffer is double-buffered by tile parity, so one barrier per tile suffices:
// a wave only rewrites a buffer after every wave has passed the barrier of
// the tile in between, which follows all reads of that buffer.
template <int N, int S>
struct Split {
    static_assert(N % S == 0 && TT % S == 0, "states and tile tokens split evenly over waves");
    static constexpr int NPW = N / S;   // states per wave
    static constexpr int TPW = TT / S;  // tokens each wave finalises per tile
};

// B and C reach the waves through LDS. A tile's B[b, t, :] and C[b, t, :]
// rows are one contiguous run of TT*N values per tensor; all lanes of the
// workgroup fetch the next tile's run a tile ahead (one or two values each,
// with the same in-order vector loads as x and delta), convert it to fp32
// and store it to LDS right before the tile's barrier. Each wave then reads
// its N/S-state slice with wave-uniform (broadcast, conflict-free) LDS reads.
// Scalar loads are avoided on purpose: their completion counter cannot be
// waited on in order, so they cannot be issued a tile ahead.
template <int N, int S>
struct BcStage {
    static constexpr int kVals = TT * N;                                // per tensor per tile
    static constexpr int kPerLane = (kVals + kWave * S - 1) / (kWave * S);
    // LDS floats per tensor: the tile's values, rounded up to whole 16-byte
    // runs so the C run starts aligned. Lanes past the values wrap around:
    // they load and store the same value as the lane kVals below them, so
    // every lane issues the same loads and stores without a branch.
    static constexpr int kSlots = (kVals + 3) / 4 * 4;
    __device__ static int slot(int q, int tid) { return (q * kWave * S + tid) % kVals; }
};

struct BcIo {
    __amdgpu_buffer_rsrc_t B, C;  // base: B[b, t0, 0] / C[b, t0, 0], extent: the chunk's rows
};

template <int N, int S, int IO, bool WANT_C = true>
__device__ __forceinline__ void fetch_bc(const BcIo& bc, int tile, int cnt,
                                         uint32_t (&braw)[BcStage<N, S>::kPerLane],
                                         uint32_t (&craw)[BcStage<N, S>::kPerLane]) {
    constexpr int esz = IO == kIoF32 ? 4 : 2;
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < BcStage<N, S>::kPerLane; ++q) {
        // values past the tile's last token are clamped onto it (in bounds, unused)
        const int idx = min(BcStage<N, S>::slot(q, tid), cnt * N - 1);
        // below 2^32 by the plan, which may exceed a signed int: unsigned math
        const uint32_t off = (static_cast<uint32_t>(tile) * (TT * N) + static_cast<uint32_t>(idx)) *
                             static_cast<uint32_t>(esz);
        braw[q] = buf_load<IO>(bc.B, off, 0);
        craw[q] = WANT_C ? buf_load<IO>(bc.C, off, 0) : 0u;
    }
}

// LDS layout of one staged tile: [tensor B, C][token j][state n], fp32,
// each tensor padded to kSlots floats.
template <int N, int S, int IO, bool WANT_C = true>
__device__ __forceinline__ void stage_bc(float* bcs, const uint32_t (&braw)[BcStage<N, S>::kPerLane],
                                         const uint32_t (&craw)[BcStage<N, S>::kPerLane]) {
    constexpr int P = BcStage<N, S>::kSlots;
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < BcStage<N, S>::kPerLane; ++q) {
        // a wrapped-around lane writes the value its twin writes
        const int idx = BcStage<N, S>::slot(q, tid);
        bcs[idx] = raw_to_f32<IO>(braw[q]);
        if constexpr (WANT_C) bcs[P + idx] = raw_to_f32<IO>(craw[q]);
    }
}

// This wave's slice of one staged row (wave-uniform LDS reads).
template <int NPW>
__device__ __forceinline__ void read_slice(const float* row, float (&out)[NPW]) {
    if constexpr (NPW % 4 == 0) {
#pragma unroll
        for (int k = 0; k < NPW; k += 4) {
            const float4 v = *reinterpret_cast<const float4*>(row + k);
            out[k] = v.x; out[k + 1] = v.y; out[k + 2] = v.z; out[k + 3] = v.w;
        }
    } else if constexpr (NPW % 2 == 0) {
#pragma unroll
        for (int k = 0; k < NPW; k += 2) {
            const float2 v = *reinterpret_cast<const float2*>(row + k);
            out[k] = v.x; out[k + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int k = 0; k < NPW; ++k) out[k] = row[k];
    }
}

// With S > 1 the per-token inputs reach the waves through LDS as well. Wave w
// fetches x, delta and z only of the tokens it finalises (j = w, w+S, ... of
// the tile), converts them once and stages (delta, delta*x) as fp32 pairs for
// every wave to read; D*x and z of those tokens stay in its registers for its
// own epilogue. Each (channel, token) is converted once, whatever S is, and a
// wave holds only TT/S tokens of prefetched inputs in VGPRs. With S == 1 the
// single wave keeps all TT tokens in registers and uses them directly.
template <int S>
struct Tile {
    uint32_t x[TT / S], dt[TT / S], z[TT / S];
};

// Delta as the recurrence uses it: the raw input plus the channel's bias,
// through softplus when SP is set. SP is a compile-time switch: a runtime
// branch here gets the main loop unswitched into two copies whose register
// allocation is worse than either alone.
template <int S, int IO, bool SP>
__device__ __forceinline__ void delta_tile(const Tile<S>& r, float bias, float (&dt)[TT / S]) {
#pragma unroll
    for (int jj = 0; jj < TT / S; ++jj) {
        const float v = raw_to_f32<IO>(r.dt[jj]) + bias;
        dt[jj] = SP ? softplus_f32(v) : v;
    }
}

// Token indices are clamped to the chunk, so the ragged last tile reads only
// tokens that exist (the clamped copies are never used).
template <int S, int IO, bool LOAD_Z>
__device__ __forceinline__ void fetch_tile(const ChunkIo& io, int tile, int w, int ntok,
                                           Tile<S>& r) {
#pragma unroll
    for (int jj = 0; jj < TT / S; ++jj) {
        const int tok = min(tile * TT + jj * S + w, ntok - 1);
        const uint32_t off = static_cast<uint32_t>(tok) * io.row_bytes;
        r.x[jj] = buf_load<IO>(io.x, io.lane_bytes, off);
        r.dt[jj] = buf_load<IO>(io.delta, io.lane_bytes, off);
        r.z[jj] = LOAD_Z ? buf_load<IO>(io.z, io.lane_bytes, off) : 0u;
    }
}

// What the wave that finishes token j of a tile keeps from staging it: x as
// fp32 (the skip term D*x is one FMA at the finish) and the gate silu(z).
// Holding these instead of the raw x and z frees the raw tile as soon as it
// is staged.
template <int S>
struct Epilogue {
    float u[TT / S], gate[TT / S];
};

// LDS layout of the staged per-token inputs: [token j][lane] float2 (delta,
// delta*x). Writes the wave's own tokens and keeps their skip terms and
// gates for its epilogue.
//
// With STAGED_SUM the wave also adds the deltas of the tile's tokens it
// stages (j < cnt: the tile's valid tokens) to its partial sum `dsum`; the S
// partials are added in wave order at the chunk's end (scan_chunk).
template <int S, int IO, bool SP, bool HAS_D, bool HAS_Z, bool STAGED_SUM = false>
__device__ __forceinline__ void stage_tokens(float2* dtdu, int w, const Tile<S>& r, float dbias,
                                             float dskip, Epilogue<S>& e, int cnt = 0,
                                             float* dsum = nullptr) {
    const int lane = threadIdx.x & (kWave - 1);
    float dt[TT / S];
    delta_tile<S, IO, SP>(r, dbias, dt);
#pragma unroll
    for (int jj = 0; jj < TT / S; ++jj) {
        const float u = raw_to_f32<IO>(r.x[jj]);
        dtdu[(jj * S + w) * kWave + lane] = make_float2(dt[jj], dt[jj] * u);
        e.u[jj] = HAS_D ? u : 0.0f;
        e.gate[jj] = HAS_Z ? silu(raw_to_f32<IO>(r.z[jj])) : 1.0f;
        if constexpr (STAGED_SUM) {
            if (jj * S + w < cnt) *dsum += dt[jj];
        }
    }
}

// The state update of tokens tile*TT + [0, cnt) for this wave's states
// (FULL: cnt == TT, compiled without per-token branches). With S > 1 the
// per-token inputs come from LDS and the readout over the wave's states is
// kept per token in part[]; with S == 1 the wave holds every state, takes
// its inputs straight from its registers (delta already activated in dtv)
// and finishes and stores each token right away. With SUM (always without
// OUTPUT) the sum of delta accumulates in dsum.
template <int N, int S, int IO, bool OUTPUT, bool SUM, bool HAS_D, bool HAS_Z, bool FULL>
__device__ __forceinline__ void compute_tile(const ChunkIo& io, const float* bcs_w,
                                             const float2* dtdu, const Tile<S>& r,
                                             const float (&dtv)[TT / S], int tile, int cnt, const float (&A2)[Split<N, S>::NPW],
                                             float (&h)[Split<N, S>::NPW], float dskip,
                                             float (&part)[TT], float& dsum) {
    constexpr int NPW = Split<N, S>::NPW;
    constexpr int P = BcStage<N, S>::kSlots;
    // Tokens are taken in groups of G: all LDS inputs of a group (B and C
    // slices, delta and delta*x) are read before any of its arithmetic, so
    // the LDS latency is paid once per group. G = 2 measured best on the
    // Mamba-2.8B layer (390.6 us against 429.8 us for G = 1 and 408 us for
    // G = 4, whose extra registers cost more than the latency they hide).
    // With S == 1 the wave already holds every state and G stays 1.
    constexpr int G = S == 1 ? 1 : (kLdsGroup < TT ? kLdsGroup : TT);
    static_assert(TT % G == 0, "groups split the tile evenly");
    constexpr int NG = TT / G;
    const int lane = threadIdx.x & (kWave - 1);
    struct Group {
        float dt[G], du[G], u[G], B[G][NPW], C[G][NPW];
    };
    auto read_group = [&](int j0, Group& q) {
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
            const int j = j0 + jj;
            q.u[jj] = 0.0f;
            if constexpr (S == 1) {
                q.dt[jj] = dtv[j];
                q.u[jj] = raw_to_f32<IO>(r.x[j]);
                q.du[jj] = q.dt[jj] * q.u[jj];
            } else {
                const float2 v = dtdu[j * kWave + lane];
                q.dt[jj] = v.x;
                q.du[jj] = v.y;
            }
            read_slice<NPW>(bcs_w + j * N, q.B[jj]);
            if constexpr (OUTPUT) read_slice<NPW>(bcs_w + P + j * N, q.C[jj]);
        }
    };
    auto compute_group = [&](int j0, const Group& q) {
        // the decays of the group's tokens first: they do not depend on the
        // state, so their exponentials are in flight before the state
        // updates consume them
        float ex[G][NPW];
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
#pragma unroll
            for (int k = 0; k < NPW; ++k) ex[jj][k] = fast_exp2(q.dt[jj] * A2[k]);
        }
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
            const int j = j0 + jj;
            part[j] = 0.0f;
            if (FULL || j < cnt) {
                const float dt = q.dt[jj], du = q.du[jj], u = q.u[jj];
                if constexpr (OUTPUT) {
                    float p = 0.0f;
#pragma unroll
                    for (int k = 0; k < NPW; ++k) {
                        h[k] = fmaf(ex[jj][k], h[k], du * q.B[jj][k]);
                        p = fmaf(q.C[jj][k], h[k], p);
                    }
                    if constexpr (S == 1) {
                        if constexpr (HAS_D) p = fmaf(dskip, u, p);
                        if constexpr (HAS_Z) p *= silu(raw_to_f32<IO>(r.z[j]));
                        // Lanes past the last channel were clamped onto channel
                        // dim-1 and computed its value bit for bit, so they store
                        // the same bits to the same address; no lane mask needed.
                        buf_store<IO>(io.y, io.lane_bytes,
                                      static_cast<uint32_t>(tile * TT + j) * io.row_bytes, p);
                    }
                    part[j] = p;
                    if constexpr (SUM) dsum += dt;
                } else {
#pragma unroll
                    for (int k = 0; k < NPW; ++k) h[k] = fmaf(ex[jj][k], h[k], du * q.B[jj][k]);
                    if constexpr (SUM) dsum += dt;
                }
            }
        }
    };
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        Group q;
        read_group(g * G, q);
        // keeps the group's reads ahead of its arithmetic: left alone, the
        // scheduler issues each token's reads just before their use and
        // every token then waits out the LDS latency (reading the next
        // group's inputs before this group's arithmetic as well measured no
        // faster and took 12-22 more registers)
        if constexpr (G > 1) __builtin_amdgcn_sched_barrier(0);
        compute_group(g * G, q);
    }
}

// Wave w finishes its tokens j = w, w+S, ... of the tile: the S partial
// readouts summed in a fixed wave order, the skip term, the gate, rounding
// and the store.
template <int S, int IO, bool HAS_D, bool HAS_Z, bool FULL>
__device__ __forceinline__ void finalize_tile(const ChunkIo& io, const float* red_tile, int w,
                                              int tile, int cnt, const Epilogue<S>& e,
                                              float dskip) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int jj = 0; jj < TT / S; ++jj) {
        const int j = jj * S + w;
        if (FULL || j < cnt) {
            const float* col = red_tile + j * kWave + lane;
            float acc = col[0];
#pragma unroll
            for (int v = 1; v < S; ++v) acc += col[v * TT * kWave];
            if constexpr (HAS_D) acc = fmaf(dskip, e.u[jj], acc);
            if constexpr (HAS_Z) acc *= e.gate[jj];
            // Lanes past the last channel were clamped onto channel dim-1 and
            // computed its value bit for bit, so they store the same bits to
            // the same address; the store needs no lane mask.
            buf_store<IO>(io.y, io.lane_bytes, static_cast<uint32_t>(tile * TT + j) * io.row_bytes,
                          acc);
        }
    }
}

// LDS of one workgroup: B/C tiles, per-token inputs and partial readouts,
// each double-buffered by tile parity. A pass without outputs (OUT false:
// the chunk summaries) has no readouts, and the smaller footprint lets more
// of its workgroups share a compute unit; only the repaired carry's second
// pass (VOTE) needs the vote flags. LDS is allocated to a workgroup in whole
// kilobytes here: the output pass of split 4 and 16 states takes exactly 26
// KB, so six of its workgroups share a compute unit's 160 KB (a few bytes
// more and only five do).
template <bool VOTE, int S>
struct VoteLds {
    int vote[2][S];  // wave w's lanes are all done
};
template <int S>
struct VoteLds<false, S> {};

template <int N, int S, bool OUT = true, bool VOTE = false>
struct ScanLds : VoteLds<VOTE, S> {
    float bcs[2][2 * BcStage<N, S>::kSlots];
    float2 dtdu[2][S > 1 ? TT * kWave : 1];
    // readout partials; the summary pass keeps only the S wave partials of
    // the delta sum here (at its end)
    float red[2][S > 1 ? (OUT ? S * TT : S) * kWave : 1];
};

// What one run over a chunk computes.
enum Pass : int {
    kPassSummary = 0,  // end state and sum of delta, no y
    kPassOutput = 1,   // y from the given entering state
    kPassLocal = 2,    // y, and the sum of delta for the chunk's decay product
    kPassFixup = 3,    // y until the entering state's weight is negligible
};

// Pass 2 of the repaired carry stops once exp2(A2 * sum of delta) is at most
// 2^-kFixupLog2 for every state of the workgroup.
constexpr float kFixupLog2 = 32.0f;

// Issue priority by progress. A SIMD's scheduler prefers the oldest of its
// ready waves, so the waves sharing it finish one after the other and the
// last ones run alone, issuing far less often than a full SIMD would. A wave
// of the chunked passes lowers its own priority (s_setprio) as it passes a
// quarter, half and three quarters of its tiles, so the waves behind are
// preferred and the SIMD's waves finish together (Mamba-130M layer, 9
// chunks: 143 -> 134 us; million-token scan 8.1 -> 7.7 ms). The single-chunk
// mixed launch keeps the default order: its whole and half waves, balanced
// per SIMD by the plan, gained nothing from it.
template <bool ON>
struct ProgressPrio {
    int b1, b2, b3;  // tile indices (even) where the priority drops
    __device__ explicit ProgressPrio(int nfull)
        : b1((nfull / 4) & ~1), b2((nfull / 2) & ~1), b3((3 * nfull / 4) & ~1) {
        if constexpr (ON) __builtin_amdgcn_s_setprio(3);
    }
    __device__ void at(int i) const {
        if constexpr (ON) {
            if (i == b1) __builtin_amdgcn_s_setprio(2);
            else if (i == b2) __builtin_amdgcn_s_setprio(1);
            else if (i == b3) __builtin_amdgcn_s_setprio(0);
        }
    }
};

// All `ntok` tokens of one chunk for one wave. Two register tiles alternate
// and swap roles without register copies. With S > 1 a tile's raw inputs
// (this wave's x, delta, z and its share of the raw B/C run) are fetched two
// tiles before the tile is computed: a raw tile is free once staged (the
// epilogue keeps D*x and silu(z) instead), so step i refills the registers
// that held tile i with tile i+2 while tile i+1's raw inputs, fetched a whole
// step earlier, are staged. With S == 1 the single wave computes from the
// raw tile itself, so it fetches one tile ahead. Fetches are unconditional
// and clamp their tiles and tokens to the chunk, and the full tiles run in
// pairs inside a loop with a single exit, so every path into a compute step
// has the same loads in flight and the waits before it stay exact. A ragged
// last tile runs once after the loop.
//
// Per tile, in order: fetch tile i+2 (S > 1) or i+1; compute tile i from LDS
// buffers i&1 and store the partial readouts; stage tile i+1's B/C and
// per-token inputs into LDS buffers (i+1)&1; barrier; finalise this wave's
// tokens of tile i. Every LDS buffer is rewritten only after a barrier that
// follows its last read.
//
// kPassFixup also votes per tile: before the barrier each wave records in
// vote[i&1] whether all its lanes have exp2(a2max * dsum) <= 2^-kFixupLog2
// (a2max: the lane's largest A2), and after it every wave reads all S votes
// and the whole workgroup leaves together once they agree; the loads still
// in flight are dropped. Without kPassFixup the steps return false at
// compile time and the loop is as before.
template <int N, int S, int IO, bool SP, int PASS, bool HAS_D, bool HAS_Z, bool PRIO = true>
__device__ __forceinline__ void scan_chunk(const ChunkIo& io, const BcIo& bcio, float dbias,
                                           int ntok, int w, int n0,
                                           ScanLds<N, S, PASS != kPassSummary, PASS == kPassFixup>& lds,
                                           const float (&A2)[Split<N, S>::NPW],
                                           float (&h)[Split<N, S>::NPW], float dskip,
                                           float a2max, float& dsum) {
    constexpr bool OUTPUT = PASS != kPassSummary;
    constexpr bool SUM = PASS != kPassOutput;
    constexpr bool FIX = PASS == kPassFixup;
    constexpr bool LOAD_Z = OUTPUT && HAS_Z;
    // The passes that only need the chunk's total delta (the summary and
    // local passes: the decay product) have each wave add only the tokens it
    // stages and combine the S partials at the end, in wave order (the same
    // order in both passes, so their decay products agree bit for bit). The
    // repaired carry's second pass keeps a running sum in every wave: its
    // vote after each tile needs it.
    constexpr bool STAGED_SUM = S > 1 && (PASS == kPassSummary || PASS == kPassLocal);
    constexpr int KP = BcStage<N, S>::kPerLane;
    const int ntiles = (ntok + TT - 1) / TT;
    const int nfull = ntok / TT;
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int AHEAD = S > 1 ? 2 : 1;  // tiles between fetching a tile and computing it
    Tile<S> ta, tb;
    Epilogue<S> ea, eb;
    uint32_t bra[KP], cra[KP], brb[KP], crb[KP];

    // bf/cf receive the B/C run fetched in this step; bs/cs hold tile i+1's,
    // staged at its end (the same registers when AHEAD == 1)
    auto step = [&](auto full_tag, int i, Tile<S>& cur, const Epilogue<S>& ec, Tile<S>& nxt,
                    Epilogue<S>& en, uint32_t (&bf)[KP], uint32_t (&cf)[KP],
                    const uint32_t (&bs)[KP], const uint32_t (&cs)[KP]) -> bool {
        constexpr bool FULL = decltype(full_tag)::value;
        const int ifetch = min(i + AHEAD, ntiles - 1);
        // The B/C run is issued first and kept first (scheduling fences), so
        // with AHEAD == 1 staging it at the end of this step waits only for
        // loads older than the next tile's token inputs.
        fetch_bc<N, S, IO, OUTPUT>(bcio, ifetch, min(TT, ntok - ifetch * TT), bf, cf);
        __builtin_amdgcn_sched_barrier(0);
        fetch_tile<S, IO, LOAD_Z>(io, ifetch, w, ntok, AHEAD == 2 ? cur : nxt);
        __builtin_amdgcn_sched_barrier(0);
        const int cnt = FULL ? TT : ntok - i * TT;
        float part[TT], dtv[TT / S];
        if constexpr (S == 1) delta_tile<S, IO, SP>(cur, dbias, dtv);
        compute_tile<N, S, IO, OUTPUT, SUM && !STAGED_SUM, HAS_D, HAS_Z, FULL>(io, lds.bcs[i & 1] + n0,
                                                                lds.dtdu[i & 1], cur, dtv, i, cnt,
                                                                A2, h, dskip, part, dsum);
        if constexpr (OUTPUT && S > 1) {
            float* mine = lds.red[i & 1] + w * TT * kWave + lane;
#pragma unroll
            for (int j = 0; j < TT; ++j) mine[j * kWave] = part[j];
        }
        if constexpr (FIX) {
            // a NaN sum compares false and keeps the lane going
            const bool done = dsum * a2max <= -kFixupLog2;
            lds.vote[i & 1][w] = __builtin_amdgcn_ballot_w64(!done) == 0 ? 1 : 0;
        }
        stage_bc<N, S, IO, OUTPUT>(lds.bcs[(i + 1) & 1], bs, cs);
        if constexpr (S > 1)
            stage_tokens<S, IO, SP, OUTPUT && HAS_D, OUTPUT && HAS_Z, STAGED_SUM>(
                lds.dtdu[(i + 1) & 1], w, nxt, dbias, dskip, en, ntok - (i + 1) * TT, &dsum);
        __syncthreads();
        if constexpr (OUTPUT && S > 1)
            finalize_tile<S, IO, HAS_D, HAS_Z, FULL>(io, lds.red[i & 1], w, i, cnt, ec, dskip);
        if constexpr (FIX) {
            int all = 1;
#pragma unroll
            for (int v = 0; v < S; ++v) all &= lds.vote[i & 1][v];
            return all != 0;
        } else {
            return false;
        }
    };
    // even steps fetch into (bra, cra) and stage (brb, crb), odd steps the
    // other way round; with AHEAD == 1 every step fetches and stages (bra, cra)
    auto even = [&](auto tag, int i) -> bool {
        if constexpr (AHEAD == 2) return step(tag, i, ta, ea, tb, eb, bra, cra, brb, crb);
        else return step(tag, i, ta, ea, tb, eb, bra, cra, bra, cra);
    };
    auto odd = [&](auto tag, int i) -> bool {
        if constexpr (AHEAD == 2) return step(tag, i, tb, eb, ta, ea, brb, crb, bra, cra);
        else return step(tag, i, tb, eb, ta, ea, bra, cra, bra, cra);
    };
    using Full = std::integral_constant<bool, true>;
    using Ragged = std::integral_constant<bool, false>;

    // prologue: tile 0's B/C and token inputs into LDS buffers 0 (and, two
    // tiles ahead, tile 1's raw inputs into the second registers)
    fetch_bc<N, S, IO, OUTPUT>(bcio, 0, min(TT, ntok), bra, cra);
    fetch_tile<S, IO, LOAD_Z>(io, 0, w, ntok, ta);
    if constexpr (AHEAD == 2) {
        const int i1 = min(1, ntiles - 1);
        fetch_bc<N, S, IO, OUTPUT>(bcio, i1, min(TT, ntok - i1 * TT), brb, crb);
        fetch_tile<S, IO, LOAD_Z>(io, i1, w, ntok, tb);
    }
    stage_bc<N, S, IO, OUTPUT>(lds.bcs[0], bra, cra);
    if constexpr (S > 1)
        stage_tokens<S, IO, SP, OUTPUT && HAS_D, OUTPUT && HAS_Z, STAGED_SUM>(
            lds.dtdu[0], w, ta, dbias, dskip, ea, ntok, &dsum);
    __syncthreads();
    const ProgressPrio<PRIO> prio(nfull);
    int i = 0;
    for (; i + 2 <= nfull; i += 2) {
        prio.at(i);
        if (even(Full{}, i)) return;
        if (odd(Full{}, i + 1)) return;
    }
    if (i < nfull) {
        if (even(Full{}, i)) return;
        if (nfull < ntiles) odd(Ragged{}, i + 1);
    } else if (nfull < ntiles) {
        even(Ragged{}, i);
    }
    if constexpr (STAGED_SUM) {
        // the waves' partial delta sums, added in wave order; the barrier
        // first lets every wave finish reading the last tile's readouts
        float* part = &lds.red[0][0];
        __syncthreads();
        part[w * kWave + lane] = dsum;
        __syncthreads();
        dsum = part[lane];
#pragma unroll
        for (int v = 1; v < S; ++v) dsum += part[v * kWave + lane];
    }
}

struct ChunkGrid {
    int64_t nblk_d;           // channel groups per batch row
    int64_t nchunks;          // chunks per sequence the grid covers
    int64_t chunk_len;        // tokens per chunk
    int64_t lead = 0;         // tokens by which sequence chunk 0 is shorter
    int64_t first_chunk = 0;  // sequence chunk of the grid's chunk 0
    int64_t seq_chunks = 1;   // chunks of the whole sequence (the last one writes hL)
    int fold = 0;             // output pass: fold the chunk summaries itself (no carry pass)
};

// Sequences of at most this many chunks skip the carry pass of the rerun
// carry: each output workgroup folds the summaries of the chunks before its
// own in its prologue (at most kFoldMaxChunks - 1 pairs per state, loaded
// together), which costs less than a launch of its own.
constexpr int64_t kFoldMaxChunks = 16;

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

// Everything one wave needs to know about its place in the launch.
struct WaveSlot {
    int64_t b, k, d;   // batch row, chunk, this lane's channel (clamped)
    int w;             // wave index inside the workgroup = state slice
    int n0;            // first state of the slice
    int ntok;          // tokens of the chunk
    float dbias;       // this lane's delta bias (0 without one)
    ChunkIo io;
    BcIo bc;
};

template <int N, int S, int IO>
__device__ __forceinline__ WaveSlot wave_slot(const ScanArgs& a, const ChunkGrid& g,
                                              int64_t blk) {
    constexpr int64_t esz = IO == kIoF32 ? 4 : 2;
    WaveSlot s;
    int64_t dblk;
    decode_block(g, blk, dblk, s.k, s.b);
    s.k += g.first_chunk;
    s.w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    s.n0 = s.w * Split<N, S>::NPW;
    const int lane = threadIdx.x & (kWave - 1);
    // lanes past the last channel work on channel dim-1 (see compute_tile)
    const int64_t d0 = dblk * kWave;
    s.d = min(d0 + lane, a.dim - 1);
    // chunk k covers [k len - lead, (k+1) len - lead): the tokens that do
    // not fill whole chunks shorten chunk 0, which the rerun carry's first
    // pass scans to its outputs while the other chunks are only summarised
    const int64_t t0 = s.k == 0 ? 0 : s.k * g.chunk_len - g.lead;
    const int64_t t1 = min(a.seqlen, (s.k + 1) * g.chunk_len - g.lead);
    s.ntok = static_cast<int>(t1 - t0);
    s.dbias = a.delta_bias != nullptr ? a.delta_bias[s.d] : 0.0f;
    const int64_t first = (s.b * a.seqlen + t0) * a.dim + d0;  // element (b, t0, d0)
    // bytes from (b, t0, d0) to the end of (b, t1-1, dim-1); below 2^32 by the plan
    const uint32_t extent = static_cast<uint32_t>(((t1 - t0) * a.dim - d0) * esz);
    s.io.row_bytes = static_cast<uint32_t>(a.dim * esz);
    s.io.lane_bytes = static_cast<uint32_t>((s.d - d0) * esz);
    s.io.x = make_rsrc(static_cast<const char*>(a.x) + first * esz, extent);
    s.io.delta = make_rsrc(static_cast<const char*>(a.delta) + first * esz, extent);
    s.io.z = make_rsrc(a.z != nullptr ? static_cast<const char*>(a.z) + first * esz : nullptr,
                       extent);
    s.io.y = make_rsrc(static_cast<const char*>(a.y) + first * esz, extent);
    const int64_t bc0 = (s.b * a.seqlen + t0) * N * esz;  // B[b, t0, 0]
    const uint32_t bc_extent = static_cast<uint32_t>((t1 - t0) * N * esz);
    s.bc.B = make_rsrc(static_cast<const char*>(a.B) + bc0, bc_extent);
    s.bc.C = make_rsrc(static_cast<const char*>(a.C) + bc0, bc_extent);
    return s;
}

// The chunk carries (end states, decay products, entering states) are laid
// out [chunk][batch row][state][channel]: the lanes of a wave hold 64
// consecutive channels, so each of its per-state reads and writes is one
// contiguous run of 256 bytes. Index of state n of channel d in chunk k;
// the next state is `dim` floats on.
__device__ __forceinline__ int64_t carry_at(const ScanArgs& a, int N, int64_t k, int64_t b,
                                            int64_t d, int n) {
    return ((k * a.batch + b) * N + n) * a.dim + d;
}

// The summary of one chunk from a zero entering state: its end state and its
// decay product exp(A * sum of delta), the pair the carry folds.
template <int N, int S, int IO, bool SP>
__device__ __forceinline__ void summary_group(const ScanArgs& a, const ChunkGrid& g,
                                              const Carry& c, int64_t blk,
                                              ScanLds<N, S, false>& lds) {
    constexpr int NPW = Split<N, S>::NPW;
    const WaveSlot s = wave_slot<N, S, IO>(a, g, blk);
    float A2[NPW], h[NPW];
    const int64_t srow = carry_at(a, N, s.k, s.b, s.d, s.n0);
#pragma unroll
    for (int q = 0; q < NPW; ++q) {
        A2[q] = a.A[s.d * N + s.n0 + q] * kLog2e;
        h[q] = 0.0f;
    }
    float dsum = 0.0f;
    scan_chunk<N, S, IO, SP, kPassSummary, false, false>(s.io, s.bc, s.dbias, s.ntok, s.w, s.n0,
                                                         lds, A2, h, 0.0f, 0.0f, dsum);
#pragma unroll
    for (int q = 0; q < NPW; ++q) {
        c.end[srow + q * a.dim] = h[q];
        c.decay[srow + q * a.dim] = fast_exp2(A2[q] * dsum);
    }
}

// Carry pass: one thread per (b, n, d) column folds the chunk summaries in
// order and writes the state entering chunks 1 .. nchunks-1. With hL (the
// repaired carry, whose pass 1 summarises the last chunk too) it folds
// through the last chunk and writes the final state at (b, d, n). The pairs are loaded kCarryBatch chunks at a time
// before they are folded, so a thread waits for memory once per batch rather
// than once per chunk (the fold itself is one FMA per chunk).
constexpr int kCarryBatch = 8;

__global__ __launch_bounds__(256) void chunk_carry_kernel(int64_t columns, int64_t nchunks,
                                                          Carry c, float* hL, int64_t dim,
                                                          int64_t nstate) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    // chunks whose pair is folded: 1 .. last - 1 (the last one only with hL)
    const int64_t last = hL != nullptr ? nchunks : nchunks - 1;
    for (int64_t col = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; col < columns;
         col += stride) {
        float H = c.end[col];  // exact end state of chunk 0
        for (int64_t k0 = 1; k0 < nchunks; k0 += kCarryBatch) {
            float P[kCarryBatch], E[kCarryBatch];
#pragma unroll
            for (int u = 0; u < kCarryBatch; ++u) {
                // clamped into range; the pairs past `last` are never used
                const int64_t k = min(k0 + u, nchunks - 1);
                P[u] = c.decay[k * columns + col];
                E[u] = c.end[k * columns + col];
            }
#pragma unroll
            for (int u = 0; u < kCarryBatch; ++u) {
                const int64_t k = k0 + u;
                if (k < nchunks) c.start[k * columns + col] = H;
                if (k < last) H = fmaf(P[u], H, E[u]);
            }
        }
        if (hL != nullptr) {
            const int64_t b = col / (nstate * dim);
            const int64_t r = col - b * nstate * dim;
            const int64_t n = r / dim;
            hL[(b * dim + (r - n * dim)) * nstate + n] = H;
        }
    }
}

// Pass 2 (or the only pass when nchunks == 1): scan each chunk from its true
// entering state and write y; the last chunk writes hL.
template <int N, int S, int IO, bool SP, bool HAS_D, bool HAS_Z, bool STORE_END = false,
          bool PRIO = true>
__device__ __forceinline__ void output_group(const ScanArgs& a, const ChunkGrid& g,
                                             const Carry& c, int64_t blk, ScanLds<N, S>& lds) {
    constexpr int NPW = Split<N, S>::NPW;
    const WaveSlot s = wave_slot<N, S, IO>(a, g, blk);
    float A2[NPW], h[NPW];
#pragma unroll
    for (int q = 0; q < NPW; ++q) A2[q] = a.A[s.d * N + s.n0 + q] * kLog2e;
    if (s.k == 0) {
#pragma unroll
        for (int q = 0; q < NPW; ++q)
            h[q] = a.h0 != nullptr ? a.h0[(s.b * a.dim + s.d) * N + s.n0 + q] : 0.0f;
    } else if (g.fold) {
        // The state entering chunk k: chunk 0's end state (exact: it started
        // from h0) folded with the pairs of chunks 1 .. k-1 in order, the
        // carry pass's arithmetic (so the same bits). The pairs of
        // kFoldBatch chunks are loaded before they are folded.
        constexpr int kFoldBatch = 4;
        const int64_t cols = a.batch * a.dim * N;
        const int64_t col = carry_at(a, N, 0, s.b, s.d, s.n0);
#pragma unroll
        for (int q = 0; q < NPW; ++q) h[q] = c.end[col + q * a.dim];
        for (int64_t j0 = 1; j0 < s.k; j0 += kFoldBatch) {
            float P[kFoldBatch][NPW], E[kFoldBatch][NPW];
#pragma unroll
            for (int u = 0; u < kFoldBatch; ++u) {
                // clamped into range; pairs from chunk k on are never used
                const int64_t row = min(j0 + u, s.k - 1) * cols + col;
#pragma unroll
                for (int q = 0; q < NPW; ++q) {
                    P[u][q] = c.decay[row + q * a.dim];
                    E[u][q] = c.end[row + q * a.dim];
                }
            }
#pragma unroll
            for (int u = 0; u < kFoldBatch; ++u) {
                if (j0 + u < s.k) {
#pragma unroll
                    for (int q = 0; q < NPW; ++q) h[q] = fmaf(P[u][q], h[q], E[u][q]);
                }
            }
        }
    } else {
        const int64_t srow = carry_at(a, N, s.k, s.b, s.d, s.n0);
#pragma unroll
        for (int q = 0; q < NPW; ++q) h[q] = c.start[srow + q * a.dim];
    }
    const float dskip = HAS_D ? a.D[s.d] : 0.0f;
    float dsum = 0.0f;
    scan_chunk<N, S, IO, SP, kPassOutput, HAS_D, HAS_Z, PRIO>(s.io, s.bc, s.dbias, s.ntok, s.w, s.n0,
                                                        lds, A2, h, dskip, 0.0f, dsum);
    if constexpr (STORE_END) {
        // chunk 0 of a cut sequence: its end state, exact since it started
        // from h0, is the state entering chunk 1 and where the fold starts
        const int64_t srow = carry_at(a, N, s.k, s.b, s.d, s.n0);
#pragma unroll
        for (int q = 0; q < NPW; ++q) c.end[srow + q * a.dim] = h[q];
    } else if (s.k == g.seq_chunks - 1 && a.hL != nullptr) {
#pragma unroll
        for (int q = 0; q < NPW; ++q) a.hL[(s.b * a.dim + s.d) * N + s.n0 + q] = h[q];
    }
}

template <int N, int S, int IO, bool SP, bool HAS_D, bool HAS_Z>
__global__ __launch_bounds__(kWave * S) __attribute__((amdgpu_waves_per_eu(S <= 2 ? 2 : 4)))
void chunk_output_kernel(ScanArgs a, ChunkGrid g, Carry c) {
    __shared__ ScanLds<N, S> lds;
    output_group<N, S, IO, SP, HAS_D, HAS_Z>(a, g, c, blockIdx.x, lds);
}

// Rerun carry, pass 1, over chunks 0 .. nchunks-2. Chunk 0 starts from h0,
// so it runs the output pass straight away: its y is final and its end state
// is the exact state entering chunk 1. The other chunks store their summary
// pairs. Pass 2 then covers chunks 1 .. nchunks-1 only, so each launch holds
// nchunks-1 layers of channel groups; the plan picks the chunk count that
// spreads those workgroups evenly over the compute units.
template <int N, int S, int IO, bool SP, bool HAS_D, bool HAS_Z>
__global__ __launch_bounds__(kWave * S) __attribute__((amdgpu_waves_per_eu(S <= 2 ? 2 : 4)))
void chunk_head_kernel(ScanArgs a, ChunkGrid g, Carry c) {
    __shared__ union {
        ScanLds<N, S> out;
        ScanLds<N, S, false> sum;
    } lds;
    const int64_t blk = blockIdx.x;
    int64_t dblk, k, b;
    decode_block(g, blk, dblk, k, b);
    if (k + g.first_chunk == 0)
        output_group<N, S, IO, SP, HAS_D, HAS_Z, true>(a, g, c, blk, lds.out);
    else
        summary_group<N, S, IO, SP>(a, g, c, blk, lds.sum);
}

// ---------------------------------------------------------------------------
// Half channel groups (single-chunk scans of split 4). A launch of G channel
// groups on C compute units leaves some units with one workgroup more than
// others unless G is a multiple of C; on the Mamba-2.8B layer (640 groups,
// 2.5 per unit) the units holding three set the time while the others idle.
// The plan can split the last groups in two halves of 32 channels each, so
// that every unit holds its share of whole groups plus at most one half.
// A half workgroup has the same 4 waves and 256 lanes as a whole one, but
// each wave holds two 32-lane rows: lanes 0..31 and 32..63 of wave w take
// state split v = 2w and 2w + 1 of 8 (N/8 states each) for the same 32
// channels. Every channel's states are spread over 8 lanes, a lane does half
// the state work of a whole group's lane, and a token's readout sums 8
// partials. Split v also owns token v of every 8-token tile: it loads,
// converts and stages that token's inputs for its 32 channels and finishes
// that token's outputs, so every (channel, token) is converted and finished
// once. The tile pipeline is the whole group's (inputs two tiles ahead, B/C
// staged in LDS, one barrier per tile, double-buffered LDS); only the token
// a lane loads or stores differs per lane, so its row offset goes into the
// per-lane buffer offset.
constexpr int kHalf = kHalfChannels;
constexpr int kSplitsHalf = kHalfSplits;

template <int N>
struct HalfLds {
    float bcs[2][2 * BcStage<N, 4>::kSlots];
    float2 dtdu[2][TT * kHalf];               // (delta, delta*x) per token and channel
    float red[2][kSplitsHalf * TT * kHalf];   // partial readouts per split, token, channel
};

template <int IO>
__device__ __forceinline__ uint32_t buf_load_lane(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (IO == kIoF32) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0);
    } else {
        return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), 0, 0);
    }
}

template <int N, int IO, bool SP, bool HAS_D, bool HAS_Z>
__device__ __forceinline__ void half_group(const ScanArgs& a, int64_t b, int64_t d0,
                                           HalfLds<N>& lds) {
    constexpr int NPS = N / kSplitsHalf;  // states per lane
    static_assert(N % kSplitsHalf == 0 && TT == kSplitsHalf, "one token per split and tile");
    constexpr int KP = BcStage<N, 4>::kPerLane;
    constexpr int P = BcStage<N, 4>::kSlots;
    constexpr int64_t esz = IO == kIoF32 ? 4 : 2;
    const int lane = threadIdx.x & (kWave - 1);
    const int ch = lane & (kHalf - 1);
    const int v = 2 * (static_cast<int>(threadIdx.x) / kWave) + (lane >> 5);
    const int n0 = v * NPS;
    // lanes past the last channel work on channel dim-1 (as in a whole group)
    const int64_t d = min(d0 + ch, a.dim - 1);
    const int64_t L = a.seqlen;
    const int ntok = static_cast<int>(L);
    const int ntiles = (ntok + TT - 1) / TT;
    const int nfull = ntok / TT;
    const float dbias = a.delta_bias != nullptr ? a.delta_bias[d] : 0.0f;
    const float dskip = HAS_D ? a.D[d] : 0.0f;
    float A2[NPS], h[NPS];
#pragma unroll
    for (int q = 0; q < NPS; ++q) {
        A2[q] = a.A[d * N + n0 + q] * kLog2e;
        h[q] = a.h0 != nullptr ? a.h0[(b * a.dim + d) * N + n0 + q] : 0.0f;
    }
    // the row from (b, 0, d0) to the end of (b, L-1, dim-1): below 2^32 bytes
    // because the plan only splits groups of single-chunk scans
    const int64_t first = b * L * a.dim + d0;
    const uint32_t extent = static_cast<uint32_t>((L * a.dim - d0) * esz);
    const uint32_t row_bytes = static_cast<uint32_t>(a.dim * esz);
    const uint32_t lane_bytes = static_cast<uint32_t>((d - d0) * esz);
    const auto rx = make_rsrc(static_cast<const char*>(a.x) + first * esz, extent);
    const auto rdt = make_rsrc(static_cast<const char*>(a.delta) + first * esz, extent);
    const auto rz = make_rsrc(a.z != nullptr ? static_cast<const char*>(a.z) + first * esz : nullptr,
                              extent);
    const auto ry = make_rsrc(static_cast<char*>(a.y) + first * esz, extent);
    BcIo bcio;
    bcio.B = make_rsrc(static_cast<const char*>(a.B) + b * L * N * esz,
                       static_cast<uint32_t>(L * N * esz));
    bcio.C = make_rsrc(static_cast<const char*>(a.C) + b * L * N * esz,
                       static_cast<uint32_t>(L * N * esz));

    struct Raw {
        uint32_t x, dt, z;
    };
    struct Epi {
        float u, gate;  // x as fp32 (skip term: one FMA at the finish), silu(z)
    };
    // this lane's token of tile `tile`, clamped to the sequence (unused copies)
    auto fetch = [&](int tile, Raw& r) {
        const int tok = min(tile * TT + v, ntok - 1);
        const uint32_t off = lane_bytes + static_cast<uint32_t>(tok) * row_bytes;
        r.x = buf_load_lane<IO>(rx, off);
        r.dt = buf_load_lane<IO>(rdt, off);
        r.z = HAS_Z ? buf_load_lane<IO>(rz, off) : 0u;
    };
    auto stage = [&](float2* dtdu, const Raw& r, Epi& e) {
        float dt = raw_to_f32<IO>(r.dt) + dbias;
        if constexpr (SP) dt = softplus_f32(dt);
        const float u = raw_to_f32<IO>(r.x);
        dtdu[v * kHalf + ch] = make_float2(dt, dt * u);
        e.u = HAS_D ? u : 0.0f;
        e.gate = HAS_Z ? silu(raw_to_f32<IO>(r.z)) : 1.0f;
    };
    auto step = [&](auto full_tag, int i, Raw& cur, const Epi& ec, Raw& nxt, Epi& en,
                    uint32_t (&bf)[KP], uint32_t (&cf)[KP], const uint32_t (&bs)[KP],
                    const uint32_t (&cs)[KP]) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int ifetch = min(i + 2, ntiles - 1);
        fetch_bc<N, 4, IO>(bcio, ifetch, min(TT, ntok - ifetch * TT), bf, cf);
        __builtin_amdgcn_sched_barrier(0);
        fetch(ifetch, cur);
        __builtin_amdgcn_sched_barrier(0);
        const int cnt = FULL ? TT : ntok - i * TT;
        const float* bcs = lds.bcs[i & 1];
        const float2* dtdu = lds.dtdu[i & 1];
        float* red = lds.red[i & 1] + v * TT * kHalf + ch;
        // tokens in pairs: both tokens' LDS inputs before their arithmetic
        struct Pair {
            float2 du[2];
            float Bq[2][NPS], Cq[2][NPS];
        };
        auto read_pair = [&](int j0, Pair& pr) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                pr.du[jj] = dtdu[(j0 + jj) * kHalf + ch];
                read_slice<NPS>(bcs + (j0 + jj) * N + n0, pr.Bq[jj]);
                read_slice<NPS>(bcs + P + (j0 + jj) * N + n0, pr.Cq[jj]);
            }
        };
        auto compute_pair = [&](int j0, const Pair& pr) {
            float ex[2][NPS];  // the pair's decays first (see compute_tile)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
                for (int q = 0; q < NPS; ++q) ex[jj][q] = fast_exp2(pr.du[jj].x * A2[q]);
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = j0 + jj;
                if (FULL || j < cnt) {
                    float p = 0.0f;
#pragma unroll
                    for (int q = 0; q < NPS; ++q) {
                        h[q] = fmaf(ex[jj][q], h[q], pr.du[jj].y * pr.Bq[jj][q]);
                        p = fmaf(pr.Cq[jj][q], h[q], p);
                    }
                    red[j * kHalf] = p;
                }
            }
        };
#pragma unroll
        for (int j0 = 0; j0 < TT; j0 += 2) {
            Pair pr;
            read_pair(j0, pr);
            __builtin_amdgcn_sched_barrier(0);
            compute_pair(j0, pr);
        }
        stage_bc<N, 4, IO>(lds.bcs[(i + 1) & 1], bs, cs);
        stage(lds.dtdu[(i + 1) & 1], nxt, en);
        __syncthreads();
        // finish this lane's token of tile i: the 8 partials in split order
        if (FULL || v < cnt) {
            const float* col = lds.red[i & 1] + v * kHalf + ch;
            float acc = col[0];
#pragma unroll
            for (int u = 1; u < kSplitsHalf; ++u) acc += col[u * TT * kHalf];
            if constexpr (HAS_D) acc = fmaf(dskip, ec.u, acc);
            if constexpr (HAS_Z) acc *= ec.gate;
            const uint32_t off = lane_bytes + static_cast<uint32_t>(i * TT + v) * row_bytes;
            if constexpr (IO == kIoF32) {
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc), ry, static_cast<int>(off),
                                                      0, 0);
            } else {
                const __bf16 hv = static_cast<__bf16>(acc);  // round to nearest even
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, hv), ry,
                                                      static_cast<int>(off), 0, 0);
            }
        }
    };

    Raw ra, rb;
    Epi ea, eb;
    uint32_t bra[KP], cra[KP], brb[KP], crb[KP];
    fetch_bc<N, 4, IO>(bcio, 0, min(TT, ntok), bra, cra);
    fetch(0, ra);
    {
        const int i1 = min(1, ntiles - 1);
        fetch_bc<N, 4, IO>(bcio, i1, min(TT, ntok - i1 * TT), brb, crb);
        fetch(i1, rb);
    }
    stage_bc<N, 4, IO>(lds.bcs[0], bra, cra);
    stage(lds.dtdu[0], ra, ea);
    __syncthreads();
    using Full = std::integral_constant<bool, true>;
    using Ragged = std::integral_constant<bool, false>;
    // even steps fetch into (ra, bra, cra) and stage (rb, brb, crb), odd steps
    // the other way round
    int i = 0;
    for (; i + 2 <= nfull; i += 2) {
        step(Full{}, i, ra, ea, rb, eb, bra, cra, brb, crb);
        step(Full{}, i + 1, rb, eb, ra, ea, brb, crb, bra, cra);
    }
    if (i < nfull) {
        step(Full{}, i, ra, ea, rb, eb, bra, cra, brb, crb);
        if (nfull < ntiles) step(Ragged{}, i + 1, rb, eb, ra, ea, brb, crb, bra, cra);
    } else if (nfull < ntiles) {
        step(Ragged{}, i, ra, ea, rb, eb, bra, cra, brb, crb);
    }
    if (a.hL != nullptr) {
#pragma unroll
        for (int q = 0; q < NPS; ++q) a.hL[(b * a.dim + d) * N + n0 + q] = h[q];
    }
}

// One launch of whole and half groups (single chunk, split 4): blocks
// [0, nwhole) are whole groups 0 .. nwhole-1 in (row, group) order, the
// blocks after them the two halves of each remaining group, placed by
// half_block_pair so that one XCD's L2 fetches the rows of x, delta and z a
// group's halves share (as neighbours on two XCDs they read those rows
// twice from HBM: +100 MB per Mamba-2.8B layer).
template <int N, int IO, bool SP, bool HAS_D, bool HAS_Z>
__global__ __launch_bounds__(kWave * 4) __attribute__((amdgpu_waves_per_eu(4)))
void chunk_mixed_kernel(ScanArgs a, ChunkGrid g, int64_t nwhole) {
    __shared__ union {
        ScanLds<N, 4> whole;
        HalfLds<N> half;
    } lds;
    const int64_t blk = blockIdx.x;
    if (blk < nwhole) {
        output_group<N, 4, IO, SP, HAS_D, HAS_Z, false, false>(a, g, Carry{nullptr, nullptr, nullptr}, blk,
                                                 lds.whole);
    } else {
        int64_t pair;
        int side;
        half_block_pair(blk - nwhole, static_cast<int64_t>(gridDim.x) - nwhole, pair, side);
        const int64_t grp = nwhole + pair;
        const int64_t d0 = (grp % g.nblk_d) * kWave + side * kHalf;
        // a second half wholly past the last channel has nothing to do (the
        // whole workgroup leaves before its first barrier)
        if (d0 >= a.dim) return;
        half_group<N, IO, SP, HAS_D, HAS_Z>(a, grp / g.nblk_d, d0, lds.half);
    }
}

// Repaired carry, pass 1: every chunk from a zero state (chunk 0 from h0)
// writes y and its (end state, decay product) pair, the last chunk's
// included.
template <int N, int S, int IO, bool SP, bool HAS_D, bool HAS_Z>
__global__ __launch_bounds__(kWave * S) __attribute__((amdgpu_waves_per_eu(S <= 2 ? 2 : 4)))
void chunk_local_kernel(ScanArgs a, ChunkGrid g, Carry c) {
    constexpr int NPW = Split<N, S>::NPW;
    __shared__ ScanLds<N, S> lds;
    const WaveSlot s = wave_slot<N, S, IO>(a, g, blockIdx.x);
    float A2[NPW], h[NPW];
    const int64_t srow = carry_at(a, N, s.k, s.b, s.d, s.n0);
#pragma unroll
    for (int q = 0; q < NPW; ++q) {
        A2[q] = a.A[s.d * N + s.n0 + q] * kLog2e;
        h[q] = (s.k == 0 && a.h0 != nullptr) ? a.h0[(s.b * a.dim + s.d) * N + s.n0 + q] : 0.0f;
    }
    const float dskip = HAS_D ? a.D[s.d] : 0.0f;
    float dsum = 0.0f;
    scan_chunk<N, S, IO, SP, kPassLocal, HAS_D, HAS_Z>(s.io, s.bc, s.dbias, s.ntok, s.w, s.n0,
                                                       lds, A2, h, dskip, 0.0f, dsum);
#pragma unroll
    for (int q = 0; q < NPW; ++q) {
        c.end[srow + q * a.dim] = h[q];
        c.decay[srow + q * a.dim] = fast_exp2(A2[q] * dsum);
    }
}

// Repaired carry, pass 2: chunks 1 .. nchunks-1 rerun from their true
// entering state and overwrite y until the entering state's weight has
// fallen below 2^-kFixupLog2 for every state of the workgroup.
template <int N, int S, int IO, bool SP, bool HAS_D, bool HAS_Z>
__global__ __launch_bounds__(kWave * S) __attribute__((amdgpu_waves_per_eu(S <= 2 ? 2 : 4)))
void chunk_fixup_kernel(ScanArgs a, ChunkGrid g, Carry c) {
    constexpr int NPW = Split<N, S>::NPW;
    __shared__ ScanLds<N, S, true, true> lds;
    const WaveSlot s = wave_slot<N, S, IO>(a, g, blockIdx.x);
    float A2[NPW], h[NPW];
    const int64_t srow = carry_at(a, N, s.k, s.b, s.d, s.n0);
    float a2max = -__builtin_inff();
    bool finite = true;
#pragma unroll
    for (int q = 0; q < NPW; ++q) {
        A2[q] = a.A[s.d * N + s.n0 + q] * kLog2e;
        h[q] = c.start[srow + q * a.dim];
        a2max = fmaxf(a2max, A2[q]);
        finite = finite && __builtin_isfinite(h[q]);
    }
    // an infinite or NaN entering state reaches every later output, as in
    // the two-pass form: its lanes never vote done
    if (!finite) a2max = __builtin_nanf("");
    const float dskip = HAS_D ? a.D[s.d] : 0.0f;
    float dsum = 0.0f;
    scan_chunk<N, S, IO, SP, kPassFixup, HAS_D, HAS_Z>(s.io, s.bc, s.dbias, s.ntok, s.w, s.n0,
                                                       lds, A2, h, dskip, a2max, dsum);
}

// ---------------------------------------------------------------------------
// Host-side dispatch over the compile-time variants.
template <int N, int S, int IO, bool SP, bool HAS_D, bool HAS_Z>
hipError_t launch_repaired(const ScanArgs& a, const ChunkGrid& g, const Carry& c,
                           int64_t columns, hipStream_t s) {
    const dim3 block(kWave * S);
    hipLaunchKernelGGL((chunk_local_kernel<N, S, IO, SP, HAS_D, HAS_Z>),
                       dim3(g.nblk_d * g.nchunks * a.batch), block, 0, s, a, g, c);
    hipLaunchKernelGGL(chunk_carry_kernel, dim3(stride_blocks(columns)), dim3(256), 0, s, columns,
                       g.nchunks, c, a.hL, a.dim, static_cast<int64_t>(N));
    ChunkGrid g2 = g;
    g2.nchunks = g.nchunks - 1;
    g2.first_chunk = 1;
    hipLaunchKernelGGL((chunk_fixup_kernel<N, S, IO, SP, HAS_D, HAS_Z>),
                       dim3(g.nblk_d * g2.nchunks * a.batch), block, 0, s, a, g2, c);
    return hipGetLastError();
}

// Rerun carry: pass 1 (chunk 0's outputs and the summaries of chunks 1 ..
// n-2), the carry fold (inside pass 2 for up to kFoldMaxChunks chunks, else
// its own launch), pass 2 (the outputs of chunks 1 .. n-1). Both passes
// describe n-1 chunks; the workspace rows keep the full n stride through
// `columns`.
template <int N, int S, int IO, bool SP, bool HAS_D, bool HAS_Z>
hipError_t launch_rerun(const ScanArgs& a, const ChunkGrid& g, const Carry& c, int64_t columns,
                        hipStream_t s) {
    const dim3 block(kWave * S);
    ChunkGrid g1 = g;
    g1.nchunks = g.seq_chunks - 1;
    const dim3 grid(g.nblk_d * g1.nchunks * a.batch);
    hipLaunchKernelGGL((chunk_head_kernel<N, S, IO, SP, HAS_D, HAS_Z>), grid, block, 0, s, a, g1, c);
    ChunkGrid g2 = g1;
    g2.first_chunk = 1;
    if (g.seq_chunks <= kFoldMaxChunks) {
        g2.fold = 1;
    } else {
        hipLaunchKernelGGL(chunk_carry_kernel, dim3(stride_blocks(columns)), dim3(256), 0, s,
                           columns, g.seq_chunks, c, nullptr, a.dim, static_cast<int64_t>(N));
    }
    hipLaunchKernelGGL((chunk_output_kernel<N, S, IO, SP, HAS_D, HAS_Z>), grid, block, 0, s, a, g2, c);
    return hipGetLastError();
}

template <int N, int S, int IO, bool SP>
hipError_t launch_scan_ns(const ScanArgs& a, const ScanPlan& plan, void* ws, hipStream_t s) {
    ChunkGrid g;
    g.nblk_d = (a.dim + kWave - 1) / kWave;
    g.nchunks = plan.nchunks;
    g.seq_chunks = plan.nchunks;
    g.chunk_len = plan.chunk_len;
    g.lead = plan.nchunks * plan.chunk_len - a.seqlen;
    Carry c{nullptr, nullptr, nullptr};
    const int64_t columns = a.batch * a.dim * N;
    if (plan.nchunks > 1) {
        float* base = static_cast<float*>(ws);
        c.start = base;
        c.end = base + plan.nchunks * columns;
        c.decay = base + 2 * plan.nchunks * columns;
    }
    const bool has_d = a.D != nullptr, has_z = a.z != nullptr;
    if constexpr (S == 4 && N % kSplitsHalf == 0) {
        if (plan.nchunks == 1 && plan.halves > 0) {
            const int64_t nwhole = g.nblk_d * a.batch - plan.halves;
            const dim3 grid(nwhole + 2 * plan.halves), block(kWave * S);
            if (has_d && has_z)
                hipLaunchKernelGGL((chunk_mixed_kernel<N, IO, SP, true, true>), grid, block, 0, s, a, g, nwhole);
            else if (has_d)
                hipLaunchKernelGGL((chunk_mixed_kernel<N, IO, SP, true, false>), grid, block, 0, s, a, g, nwhole);
            else if (has_z)
                hipLaunchKernelGGL((chunk_mixed_kernel<N, IO, SP, false, true>), grid, block, 0, s, a, g, nwhole);
            else
                hipLaunchKernelGGL((chunk_mixed_kernel<N, IO, SP, false, false>), grid, block, 0, s, a, g, nwhole);
            return hipGetLastError();
        }
    }
    if (plan.nchunks > 1 && plan.carry == kCarryRepair) {
        if (has_d && has_z) return launch_repaired<N, S, IO, SP, true, true>(a, g, c, columns, s);
        if (has_d) return launch_repaired<N, S, IO, SP, true, false>(a, g, c, columns, s);
        if (has_z) return launch_repaired<N, S, IO, SP, false, true>(a, g, c, columns, s);
        return launch_repaired<N, S, IO, SP, false, false>(a, g, c, columns, s);
    }
    if (plan.nchunks > 1) {
        if (has_d && has_z) return launch_rerun<N, S, IO, SP, true, true>(a, g, c, columns, s);
        if (has_d) return launch_rerun<N, S, IO, SP, true, false>(a, g, c, columns, s);
        if (has_z) return launch_rerun<N, S, IO, SP, false, true>(a, g, c, columns, s);
        return launch_rerun<N, S, IO, SP, false, false>(a, g, c, columns, s);
    }
    const dim3 grid(g.nblk_d * a.batch), block(kWave * S);
    if (has_d && has_z)
        hipLaunchKernelGGL((chunk_output_kernel<N, S, IO, SP, true, true>), grid, block, 0, s, a, g, c);
    else if (has_d)
        hipLaunchKernelGGL((chunk_output_kernel<N, S, IO, SP, true, false>), grid, block, 0, s, a, g, c);
    else if (has_z)
        hipLaunchKernelGGL((chunk_output_kernel<N, S, IO, SP, false, true>), grid, block, 0, s, a, g, c);
    else
        hipLaunchKernelGGL((chunk_output_kernel<N, S, IO, SP, false, false>), grid, block, 0, s, a, g, c);
    return hipGetLastError();
}

// The state split S is a compile-time parameter; every N supports S = 1 and
// N = 16, 8 and 4 also support the splits that divide them (up to 8).
template <int N, int IO, bool SP>
hipError_t launch_scan_n(const ScanArgs& a, const ScanPlan& plan, void* ws, hipStream_t s) {
    switch (plan.state_split) {
        case 1: return launch_scan_ns<N, 1, IO, SP>(a, plan, ws, s);
        case 2: if constexpr (N % 2 == 0 && (N == 4 || N == 8 || N == 16)) return launch_scan_ns<N, 2, IO, SP>(a, plan, ws, s); break;
        case 4: if constexpr (N % 4 == 0 && (N == 4 || N == 8 || N == 16)) return launch_scan_ns<N, 4, IO, SP>(a, plan, ws, s); break;
        case 8: if constexpr (N % 8 == 0 && (N == 8 || N == 16)) return launch_scan_ns<N, 8, IO, SP>(a, plan, ws, s); break;
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

template <int IO, bool SP, int PART>
hipError_t launch_scan_variant(const ScanArgs& a, const ScanPlan& p, void* ws, hipStream_t s) {
    // PART 0 holds dstate 1..8, PART 1 dstate 9..16 (two objects per variant)
    switch (a.dstate) {
#define MAMBA_CASE(n)                                                    \
    case n:                                                              \
        if constexpr ((n > 8) == (PART == 1)) return launch_scan_n<n, IO, SP>(a, p, ws, s); \
        break;
        MAMBA_CASE(1) MAMBA_CASE(2) MAMBA_CASE(3) MAMBA_CASE(4) MAMBA_CASE(5) MAMBA_CASE(6)
        MAMBA_CASE(7) MAMBA_CASE(8) MAMBA_CASE(9) MAMBA_CASE(10) MAMBA_CASE(11) MAMBA_CASE(12)
        MAMBA_CASE(13) MAMBA_CASE(14) MAMBA_CASE(15) MAMBA_CASE(16)
#undef MAMBA_CASE
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace mamba
