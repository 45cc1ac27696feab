// Backward pass of the selective scan by recomputation (page "Mamba and
// State Space Models", world.lapla.si, section "A Scan on the Chip": the
// states that training's backward pass needs are computed again instead of
// being stored).
//
// For the loss sum(dy * y) + sum(dhL * hL), with g_t = dy_t * silu(z_t) and
// the adjoint of the state
//     lam_t[n] = C_t[n] g_t + Abar_{t+1}[n] lam_{t+1}[n],   lam_L = dhL,
// one step h_t = Abar_t h_{t-1} + dt_t B_t x_t, Abar_t = exp(dt_t A), gives
//     dx_t   = D g_t + sum_n lam_t dt_t B_t          d dt_t = sum_n lam_t (A Abar_t h_{t-1} + B_t x_t)
//     dA    += lam_t dt_t Abar_t h_{t-1}             dB_t  += lam_t dt_t x_t   (over channels)
//     dC_t  += g_t h_t          (over channels)      dD    += g_t x_t
//     dz_t   = dy_t p_t silu'(z_t), p_t = C_t.h_t + D x_t
//     dh0    = Abar_0 lam_0;  with dt = softplus(v): d delta = d dt sigmoid(v).
//
// Work plan. One workgroup per (batch row, 64-channel group); its
// ceil(N/4) waves split the states, 4 per wave (padded with inert states:
// A = B = C = 0). (1) It runs forward over the whole sequence in tiles of 8
// tokens and writes the state entering every tile to the workspace: the
// checkpoints, 4 B per state and tile. (2) It takes the tiles from last to
// first, carrying lam in registers: it reads the tile's checkpoint,
// recomputes the tile's 8 states per lane into registers, keeping the
// tile's decay factors too (whole groups in LDS, half groups in registers),
// so the walk back does not evaluate them again, and walks the tile
// backwards. Walking back, the adjoint is
// carried as m = Abar lam, what a token hands to the one before it: then
// lam_t = C_t g_t + m is one FMA, and with lb = sum_n lam B the per-state
// work is 9 operations (dx = D g + dt lb, d dt = sum_n A lam Abar h_{t-1} +
// x lb). A sequence cut into chunks runs (1) for every chunk in a launch of
// its own, from zero states, and (2) after the chunk carries are folded.
// Tokens past the end of the sequence are staged as inert ones (delta = x =
// g = 0, zero B and C), so the forward loops need no per-token test. Sums over
// states (dx, d dt, p) go through LDS to the wave that finishes the token;
// sums over channels (dB, dC) are reduced inside the wave by a butterfly of
// lane exchanges that leaves one finished (token, state) sum in each lane,
// written as this group's partial. (3) Small kernels add the partials over
// channel groups (dB, dC) and batch rows (dA, dD, d bias) in a fixed order,
// so results are bitwise reproducible.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace mamba {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kBT = 8;                         // tokens per tile
#ifndef MAMBA_BWD_AHEAD
#define MAMBA_BWD_AHEAD 4
#endif
constexpr int kAhead = MAMBA_BWD_AHEAD;        // tiles in flight in the forward passes
constexpr int kNpw = 4;                        // states per wave
constexpr int kVals = 2 * kBT * kNpw;          // dB and dC terms per lane per tile
static_assert(kVals == kWave, "the butterfly leaves exactly one sum per lane");

// One slot per (wave, token) of a tile: first the decay factors
// exp(dt A) of the wave's states that the tile's recomputation evaluates
// (kNpw per lane, lane-major), then, once the wave walking backwards has
// read a token's factors, its three partial sums over states for that token
// (dx, d dt, C.h; kWave each). A slot is only ever written by its own wave,
// and the sums it writes depend on the factors it read there, so the read
// comes first.
constexpr int kSlot = kNpw * kWave;
static_assert(3 * kWave <= kSlot, "the partial sums fit in the slot of the factors");

// The staged tile (all a forward pass or an adjoint summary needs, 7 KB
// for 4 waves), and with the slots the whole walk back's LDS.
template <int S>
struct BwdLdsIn {
    float2 dtx[kBT][kWave];                    // (delta as used, x) per token and channel
    float g[kBT][kWave];                       // dy * silu(z)
    alignas(16) float bc[2][kBT][kNpw * S];    // B and C rows of the tile, padded states 0
};

template <int S>
struct BwdLds : BwdLdsIn<S> {
    alignas(16) float slot[S][kBT][kSlot];
};

// What the wave that finishes token j keeps from staging.
struct Own {
    float dy, z, v, x;
};

struct Place {
    int64_t b, d;      // batch row, this lane's channel (clamped to dim-1)
    int64_t grp;       // 64-channel group
    bool valid;        // lane maps to a real channel
    int w, n0;         // wave, first state of its slice
    float dbias;
};

__device__ __forceinline__ float sigmoid_f32(float v) {
    return fast_rcp(1.0f + fast_exp2(-v * kLog2e));
}

// Issue priority by progress. The scheduler prefers the oldest ready wave of
// a SIMD, so its waves finish one after the other and the last ones run
// alone; each wave here lowers its own priority (s_setprio) as it gets
// through its work so that the waves behind are preferred and all finish
// together. Priority 3 for the forward phase, then 2, 1 and 0 over thirds of
// the walk back.
#ifndef MAMBA_BWD_PRIO
#define MAMBA_BWD_PRIO 1
#endif
__device__ __forceinline__ void set_prio(int p) {
    if constexpr (MAMBA_BWD_PRIO) {
        if (p >= 3) __builtin_amdgcn_s_setprio(3);
        else if (p == 2) __builtin_amdgcn_s_setprio(2);
        else if (p == 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
    }
}

// Priority `top` at the first of n tiles, one lower after each of `top`
// equal parts (`top` 2: thirds).
struct PrioSteps {
    int64_t b1, b2, b3;
    __device__ PrioSteps(int64_t n, int top)
        : b1(top >= 2 ? n / (top + 1) : n), b2(top >= 2 ? 2 * n / (top + 1) : n),
          b3(top >= 3 ? 3 * n / (top + 1) : n) {}
    __device__ void at(int64_t done, int top) const {
        if (done == 0) set_prio(top);
        else if (done == b1) set_prio(top - 1);
        else if (done == b2) set_prio(top - 2);
        else if (done == b3) set_prio(top - 3);
    }
};

// Raw inputs of one tile as this thread stages them: the tokens j = w,
// w+S, ... of the tile for its lane's channel, one element of the tile's B
// and C rows (2 * kBT * 4S elements over 64S threads) and, walking
// backwards, the tile's checkpointed entering state of the lane's states.
// Loaded a tile ahead so the loads are in flight while the previous tile
// computes. Every load is issued unconditionally with its token and state
// clamped into range (the clamped values are never used): conditional loads
// leave the compiler unable to count the loads in flight, and the wait
// before the first use of an older load then also waits for these.
template <int S>
struct TileRaw {
    static constexpr int OW = (kBT + S - 1) / S;
    uint32_t x[OW], dl[OW], dy[OW], z[OW];
    uint32_t bc;
    float he[kNpw];
    float dp;   // sum of delta over the chunk before the tile (chunked walk only)
};

// Checkpoints are laid out [tile][batch row][group of 4 states][channel][4]:
// the 64 lanes of a wave (64 channels, one group of states) write and read
// one tile's checkpoint as 1 KB of contiguous memory, 16 bytes per lane.
// Index of the checkpoint of states n0 .. of channel d (n0 % 4 plus the
// count read stays within the group).
__device__ __forceinline__ int64_t tent_index(const ScanArgs& f, int64_t tile, int64_t b, int64_t d,
                                              int n0) {
    const int64_t groups = (f.dstate + 3) / 4;
    return (((tile * f.batch + b) * groups + n0 / 4) * f.dim + d) * 4 + (n0 & 3);
}

// The per-group dB/dC partials are laid out [dB|dC][slot][batch row][group
// of 4 states][token][4], `per` floats per slot: the 32 sums a wave holds
// for one of them after its butterfly (8 tokens x 4 states) are 128
// contiguous bytes. Index within a slot of (row b, token t, state n).
__device__ __forceinline__ int64_t bc_index(const ScanArgs& f, int64_t b, int64_t t, int n) {
    return ((b * ((f.dstate + 3) / 4) + n / 4) * f.seqlen + t) * 4 + (n & 3);
}

__device__ __forceinline__ int64_t bc_slot_floats(const ScanArgs& f) {
    return f.batch * ((f.dstate + 3) / 4) * f.seqlen * 4;
}

template <int S, int IO, bool HAS_Z, bool WANT_G, bool CORR = false, bool WANT_H = WANT_G>
__device__ __forceinline__ void fetch_tile(const BwdArgs& a, const Place& pl, const float* tent,
                                           int64_t tile, int cnt, TileRaw<S>& r,
                                           const float* dpre = nullptr) {
    const ScanArgs& f = a.fwd;
    const int64_t t0 = tile * kBT;
#pragma unroll
    for (int jj = 0; jj < TileRaw<S>::OW; ++jj) {
        const int j = min(jj * S + pl.w, cnt - 1);
        const int64_t idx = (pl.b * f.seqlen + t0 + j) * f.dim + pl.d;
        r.x[jj] = load_raw<IO>(f.x, idx);
        r.dl[jj] = load_raw<IO>(f.delta, idx);
        if constexpr (WANT_G) {
            r.dy[jj] = load_raw<IO>(a.dy, idx);
            r.z[jj] = HAS_Z ? load_raw<IO>(f.z, idx) : 0u;
        }
    }
    constexpr int NP = kNpw * S;
    const int e = threadIdx.x;  // exactly one B or C element per thread
    const int which = e / (kBT * NP);
    const int rr = e - which * kBT * NP;
    const int j = min(rr / NP, cnt - 1);
    const int n = min(rr % NP, f.dstate - 1);
    r.bc = load_raw<IO>(which ? f.C : f.B, (pl.b * f.seqlen + t0 + j) * f.dstate + n);
    if constexpr (WANT_H) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(tent + tent_index(f, tile, pl.b, pl.d, pl.n0));
#pragma unroll
        for (int q = 0; q < kNpw; ++q) r.he[q] = v[q];
        if constexpr (CORR) r.dp = dpre[(tile * f.batch + pl.b) * f.dim + pl.d];
    }
}

// Stage a fetched tile: wave w converts its tokens j = w, w+S, ... (delta
// activated once per (channel, token)) and every thread its B or C element.
template <int S, int IO, bool SP, bool HAS_Z, bool WANT_G>
__device__ __forceinline__ void put_tile(const TileRaw<S>& r, const Place& pl, BwdLdsIn<S>& lds,
                                         int cnt, int nstate, Own (&own)[(kBT + S - 1) / S]) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int jj = 0; jj < TileRaw<S>::OW; ++jj) {
        const int j = jj * S + pl.w;
        if (j < cnt) {
            float xf = raw_to_f32<IO>(r.x[jj]);
            const float v = raw_to_f32<IO>(r.dl[jj]) + pl.dbias;
            const float dt = SP ? softplus_f32(v) : v;
            if (!pl.valid) xf = 0.0f;  // a clamped lane contributes nothing
            lds.dtx[j][lane] = make_float2(dt, xf);
            if constexpr (WANT_G) {
                const float dyf = raw_to_f32<IO>(r.dy[jj]);
                const float zf = HAS_Z ? raw_to_f32<IO>(r.z[jj]) : 0.0f;
                float gg = HAS_Z ? dyf * silu(zf) : dyf;
                if (!pl.valid) gg = 0.0f;
                lds.g[j][lane] = gg;
                own[jj] = Own{dyf, zf, v, xf};
            }
        } else if (j < kBT) {
            // a token past the end of the sequence: inert (delta = x = g = 0
            // and zero B, C rows leave the state and every sum unchanged)
            lds.dtx[j][lane] = make_float2(0.0f, 0.0f);
            if constexpr (WANT_G) lds.g[j][lane] = 0.0f;
        }
    }
    constexpr int NP = kNpw * S;
    const int e = threadIdx.x;
    const int which = e / (kBT * NP);
    const int rr = e - which * kBT * NP;
    const bool in = rr / NP < cnt && rr % NP < nstate;   // padding states and tokens read as 0
    lds.bc[which][rr / NP][rr % NP] = in ? raw_to_f32<IO>(r.bc) : 0.0f;
}

// Sum of each of the 64 values over the 64 lanes. At the step of distance
// k, pairs (vals[2i], vals[2i+1]) are folded into vals[i]: lanes with bit k
// clear keep the first value and add their partner's (lane ^ k) copy of it,
// lanes with bit k set the second. After the steps k = 32, 16, ..., 1, lane l
// holds the full sum of the value whose index is l with its 6 bits reversed.
// All exchanges stay in the VALU: for k = 32 and 16 one lane swap of the pair
// (v_permlane32_swap / v_permlane16_swap exchange the upper half of the
// first register's 32- or 16-lane blocks with the lower half of the
// second's) leaves each lane exactly its own kept value and its partner's,
// so their sum is the step; for k <= 8 DPP row shifts bring lane l + k and
// l - k within the 16-lane row.
template <int K, int M>
__device__ __forceinline__ void fold_dpp(float (&vals)[M], int cnt, int lane) {
    const bool hi = (lane & K) != 0;
    for (int i = 0; i < cnt; ++i) {
        const float a = vals[2 * i], b = vals[2 * i + 1];
        const float up = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x100 + K, 0xf, 0xf, false));
        const float dn = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(b), 0x110 + K, 0xf, 0xf, false));
        vals[i] = hi ? b + dn : a + up;   // row_shl:K reads lane l + K, row_shr:K lane l - K
    }
}

__device__ __forceinline__ float lane_sums(float (&vals)[kVals]) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(vals[2 * i]),
                                                        __float_as_uint(vals[2 * i + 1]), false, false);
        vals[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(vals[2 * i]),
                                                        __float_as_uint(vals[2 * i + 1]), false, false);
        vals[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    fold_dpp<8>(vals, 8, lane);
    fold_dpp<4>(vals, 4, lane);
    fold_dpp<2>(vals, 2, lane);
    fold_dpp<1>(vals, 1, lane);
    return vals[0];
}

// The same over the 32 lanes of each half of the wave (the rows of a half
// group, which hold different states): 32 values, steps k = 16, ..., 1; lane
// l holds the sum of value reverse5(l mod 32) over its 32-lane half.
__device__ __forceinline__ float lane_sums32(float (&vals)[kWave / 2]) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(vals[2 * i]),
                                                        __float_as_uint(vals[2 * i + 1]), false, false);
        vals[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    fold_dpp<8>(vals, 8, lane);
    fold_dpp<4>(vals, 4, lane);
    fold_dpp<2>(vals, 2, lane);
    fold_dpp<1>(vals, 1, lane);
    return vals[0];
}

__device__ __forceinline__ int reverse5(int l) {
    return ((l & 1) << 4) | ((l & 2) << 2) | (l & 4) | ((l & 8) >> 2) | ((l & 16) >> 4);
}

__device__ __forceinline__ int reverse6(int l) {
    return ((l & 1) << 5) | ((l & 2) << 3) | ((l & 4) << 1) | ((l & 8) >> 1) | ((l & 16) >> 3) |
           ((l & 32) >> 5);
}

// Workspace pointers of the main kernel. part_bc holds nslots partial dB/dC
// slots per (row, token, state): slot g for channel group g (its first half
// when split), slot ngroups + g for the second half of a split group g.
struct BwdWs {
    float* tent;
    float* part_bc;
    float* part_a;        // [chunk][b][d][n]
    float* part_d;        // [chunk][b][d]
    float* part_bias;     // [chunk][b][d]
    int64_t nslots;
    // A sequence cut into nchunks chunks of chunk_len tokens (one chunk:
    // chunk_len covers the whole sequence). hin[c] is the state entering
    // chunk c >= 1 and rho[nchunks - 1 - c] the adjoint entering chunk
    // c <= nchunks - 2 from its right, Abar_{t1} lam_{t1} with t1 the first
    // token after the chunk; both [.][b][d][n].
    int64_t nchunks;
    int64_t chunk_len;
    const float* hin;
    const float* rho;
    // the split chunked plan: the forward pass from zero states writes each
    // chunk's end state and decay product (chunks 0 .. nchunks-2) for the
    // fold, and per tile the sum of delta over the chunk before it
    float* fend;
    float* fdecay;
    float* dpre;
};

// What a whole-group workgroup runs: the forward pass and the walk back (a
// whole sequence), the forward pass alone from a zero state, or the walk
// back alone over checkpoints that the chunk's entering state still has to
// be added to (a chunked sequence, whose forward passes run in an earlier
// launch).
enum BwdMode { kBwdBoth = 0, kBwdForward = 1, kBwdWalk = 2 };

// Place of a whole-group thread: batch row and channel group from the
// workgroup's index within its chunk, its wave's states, its channel.
__device__ __forceinline__ Place make_place(const ScanArgs& f, int64_t ngroups, int64_t in_chunk) {
    const int lane = threadIdx.x & (kWave - 1);
    Place pl;
    pl.grp = in_chunk % ngroups;
    pl.b = in_chunk / ngroups;
    pl.w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    pl.n0 = pl.w * kNpw;
    const int64_t d_raw = pl.grp * kWave + lane;
    pl.valid = d_raw < f.dim;
    pl.d = pl.valid ? d_raw : f.dim - 1;
    pl.dbias = f.delta_bias != nullptr ? f.delta_bias[pl.d] : 0.0f;
    return pl;
}

template <int S, int IO, bool SP, bool HAS_D, bool HAS_Z, int MODE = kBwdBoth, class LDS>
__device__ __forceinline__ void bwd_whole_group(const BwdArgs& a, int64_t ngroups, int64_t blk,
                                                const BwdWs& ws, LDS& lds) {
    constexpr int OW = (kBT + S - 1) / S;
    float* const tent = ws.tent;
    float* const part_bc = ws.part_bc;
    float* const part_a = ws.part_a;
    float* const part_d = ws.part_d;
    float* const part_bias = ws.part_bias;
    const ScanArgs& f = a.fwd;
    const int N = f.dstate;
    const int64_t L = f.seqlen;
    const int lane = threadIdx.x & (kWave - 1);

    // block -> (chunk, batch row, channel group); the chunk's tiles
    const int64_t rows = f.batch * ngroups;
    const int64_t chunk = blk / rows;
    const int64_t in_chunk = blk - chunk * rows;
    const bool last_chunk = chunk == ws.nchunks - 1;
    const int64_t i_first = chunk * (ws.chunk_len / kBT);
    const int64_t i_end = last_chunk ? (L + kBT - 1) / kBT : i_first + ws.chunk_len / kBT;
    const Place pl = make_place(f, ngroups, in_chunk);
    const float dskip = HAS_D ? f.D[pl.d] : 0.0f;

    // the adjoint entering the chunk from its right: dhL for the last chunk
    const int64_t col0 = (pl.b * f.dim + pl.d) * N;
    const float* lam_in = last_chunk ? a.dhL
                                     : ws.rho + (ws.nchunks - 1 - chunk) * f.batch * f.dim * N;
    bool sv[kNpw];      // state exists (not padding)
    // m: Abar lam of the token after the one being walked (what that token
    // hands back), at the chunk's end the adjoint taken in from the right
    float A[kNpw], A2[kNpw], m[kNpw], dA[kNpw];
#pragma unroll
    for (int q = 0; q < kNpw; ++q) {
        const int n = pl.n0 + q;
        sv[q] = n < N;
        A[q] = sv[q] ? f.A[pl.d * N + n] : 0.0f;
        A2[q] = A[q] * kLog2e;
        m[q] = (sv[q] && lam_in != nullptr) ? lam_in[col0 + n] : 0.0f;
        dA[q] = 0.0f;
    }
    float dD_acc = 0.0f, dbias_acc = 0.0f;
    Own own[OW];

    // (1) forward over the chunk from its entering state (alone: from a zero
    // state after chunk 0), keeping the state entering every tile in the
    // workspace (only real lanes and states write)
    if constexpr (MODE != kBwdWalk) {
        const float* h_in = chunk == 0 ? f.h0
                          : MODE == kBwdForward ? nullptr
                                                : ws.hin + chunk * f.batch * f.dim * N;
        float h[kNpw];
#pragma unroll
        for (int q = 0; q < kNpw; ++q)
            h[q] = (sv[q] && h_in != nullptr) ? h_in[col0 + pl.n0 + q] : 0.0f;
        float dsum = 0.0f;
        // tiles are fetched kAhead ahead: the pass does little arithmetic per
        // tile, so one tile of it does not cover the latency of HBM
        TileRaw<S> raw[kAhead];
#pragma unroll
        for (int u = 0; u < kAhead; ++u) {
            const int64_t nx = min(i_first + u, i_end - 1);
            fetch_tile<S, IO, HAS_Z, false>(a, pl, tent, nx,
                                            static_cast<int>(min<int64_t>(kBT, L - nx * kBT)), raw[u]);
        }
        set_prio(3);
        for (int64_t i0 = i_first; i0 < i_end; i0 += kAhead) {
#pragma unroll
            for (int u = 0; u < kAhead; ++u) {
                const int64_t i = i0 + u;
                if (i >= i_end) break;
                const int64_t t0 = i * kBT;
                const int cnt = static_cast<int>(min<int64_t>(kBT, L - t0));
                if (pl.valid) {
                    // padding states hold zero
                    *reinterpret_cast<f32x4*>(tent + tent_index(f, i, pl.b, pl.d, pl.n0)) =
                        f32x4{h[0], h[1], h[2], h[3]};
                    if constexpr (MODE == kBwdForward)
                        if (pl.w == 0) ws.dpre[(i * f.batch + pl.b) * f.dim + pl.d] = dsum;
                }
                put_tile<S, IO, SP, HAS_Z, false>(raw[u], pl, lds, cnt, N, own);
                __syncthreads();
                {
                    // the last tiles fetch the last one again (unused)
                    const int64_t nx = min(i + kAhead, i_end - 1);
                    fetch_tile<S, IO, HAS_Z, false>(a, pl, tent, nx,
                                                    static_cast<int>(min<int64_t>(kBT, L - nx * kBT)),
                                                    raw[u]);
                }
#pragma unroll
                for (int j0 = 0; j0 < kBT; j0 += 2) {
                    float2 v[2];
                    f32x4 bq[2];
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        v[jj] = lds.dtx[j0 + jj][lane];
                        bq[jj] = *reinterpret_cast<const f32x4*>(&lds.bc[0][j0 + jj][pl.n0]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        const float du = v[jj].x * v[jj].y;
                        if constexpr (MODE == kBwdForward) dsum += v[jj].x;
#pragma unroll
                        for (int q = 0; q < kNpw; ++q)
                            h[q] = fmaf(fast_exp2(v[jj].x * A2[q]), h[q], du * bq[jj][q]);
                    }
                }
                __syncthreads();
            }
        }
        if constexpr (MODE == kBwdForward) {
            // the chunk's summary for the fold: end state from the zero (or
            // initial) state and decay product
            if (!last_chunk && pl.valid) {
                const int64_t at = chunk * f.batch * f.dim * N + col0 + pl.n0;
#pragma unroll
                for (int q = 0; q < kNpw; ++q) {
                    if (sv[q]) {
                        ws.fend[at + q] = h[q];
                        ws.fdecay[at + q] = fast_exp2(A2[q] * dsum);
                    }
                }
            }
            return;
        }
    }

    // (2) the tiles in reverse. Walking alone, a chunk after the first adds
    // its entering state, decayed to the tile, to each checkpoint. (Not
    // compiled for the forward pass alone, whose LDS has no slots.)
    if constexpr (MODE != kBwdForward) {
        constexpr bool CORR = MODE == kBwdWalk;
        float hin[kNpw];
#pragma unroll
        for (int q = 0; q < kNpw; ++q)
            hin[q] = (CORR && chunk > 0 && sv[q] && pl.valid)
                         ? ws.hin[chunk * f.batch * f.dim * N + col0 + pl.n0 + q]
                         : 0.0f;
        float h[kNpw];
        TileRaw<S> raw;
        fetch_tile<S, IO, HAS_Z, true, CORR>(a, pl, tent, i_end - 1,
                                             static_cast<int>(min<int64_t>(kBT, L - (i_end - 1) * kBT)),
                                             raw, ws.dpre);
        const PrioSteps prio(i_end - i_first, 2);
        for (int64_t i = i_end - 1; i >= i_first; --i) {
            prio.at(i_end - 1 - i, 2);
            const int64_t t0 = i * kBT;
            const int cnt = static_cast<int>(min<int64_t>(kBT, L - t0));
            // the tile's entering state; a lane past the last channel starts
            // from zero (its x and g are zero too, so it contributes nothing)
            float he[kNpw], hs[kBT][kNpw];
#pragma unroll
            for (int q = 0; q < kNpw; ++q) he[q] = (pl.valid && sv[q]) ? raw.he[q] : 0.0f;
            if constexpr (CORR) {
                if (chunk > 0) {
#pragma unroll
                    for (int q = 0; q < kNpw; ++q) he[q] = fmaf(fast_exp2(A2[q] * raw.dp), hin[q], he[q]);
                }
            }
            put_tile<S, IO, SP, HAS_Z, true>(raw, pl, lds, cnt, N, own);
            __syncthreads();
            // the chunk's first tile fetches itself again (unused)
            {
                const int64_t pv = i > i_first ? i - 1 : i_first;
                fetch_tile<S, IO, HAS_Z, true, CORR>(a, pl, tent, pv,
                                                     static_cast<int>(min<int64_t>(kBT, L - pv * kBT)),
                                                     raw, ws.dpre);
            }

#pragma unroll
            for (int q = 0; q < kNpw; ++q) h[q] = he[q];
#pragma unroll
            for (int j0 = 0; j0 < kBT; j0 += 2) {
                float2 v[2];
                f32x4 bq[2];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    v[jj] = lds.dtx[j0 + jj][lane];
                    bq[jj] = *reinterpret_cast<const f32x4*>(&lds.bc[0][j0 + jj][pl.n0]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int j = j0 + jj;
                    const float du = v[jj].x * v[jj].y;
                    f32x4 ev;
#pragma unroll
                    for (int q = 0; q < kNpw; ++q) {
                        ev[q] = fast_exp2(v[jj].x * A2[q]);
                        h[q] = fmaf(ev[q], h[q], du * bq[jj][q]);
                    }
                    reinterpret_cast<f32x4*>(lds.slot[pl.w][j])[lane] = ev;
#pragma unroll
                    for (int q = 0; q < kNpw; ++q) hs[j][q] = h[q];
                }
            }

            // dB and dC terms: set token by token (zero past the sequence, in
            // the branch only partial tiles take)
            float vals[kVals];
#pragma unroll
            for (int j1 = kBT - 1; j1 >= 0; j1 -= 2) {
              // the LDS inputs of tokens j1 and j1 - 1 are read before either
              // token's arithmetic (as in the forward kernel)
              float2 vv[2];
              float gq[2];
              f32x4 bq[2], cq[2], eq[2];
#pragma unroll
              for (int jj = 0; jj < 2; ++jj) {
                  vv[jj] = lds.dtx[j1 - jj][lane];
                  gq[jj] = lds.g[j1 - jj][lane];
                  bq[jj] = *reinterpret_cast<const f32x4*>(&lds.bc[0][j1 - jj][pl.n0]);
                  cq[jj] = *reinterpret_cast<const f32x4*>(&lds.bc[1][j1 - jj][pl.n0]);
                  eq[jj] = reinterpret_cast<const f32x4*>(lds.slot[pl.w][j1 - jj])[lane];
              }
              __builtin_amdgcn_sched_barrier(0);
#pragma unroll
              for (int jj = 0; jj < 2; ++jj) {
                const int j = j1 - jj;
                if (j < cnt) {
                    const float dt = vv[jj].x, x = vv[jj].y;
                    const float gg = gq[jj];
                    const float dtx = dt * x;
                    float lb = 0.0f, dap = 0.0f, pp = 0.0f;
#pragma unroll
                    for (int q = 0; q < kNpw; ++q) {
                        const float Bq = bq[jj][q];
                        const float Cq = cq[jj][q];
                        const float lam = fmaf(Cq, gg, m[q]);
                        const float hprev = j > 0 ? hs[j > 0 ? j - 1 : 0][q] : he[q];
                        m[q] = eq[jj][q] * lam;
                        const float le = m[q] * hprev;   // lam Abar h_{t-1}
                        dA[q] = fmaf(dt, le, dA[q]);
                        dap = fmaf(A[q], le, dap);
                        lb = fmaf(lam, Bq, lb);
                        pp = fmaf(Cq, hs[j][q], pp);
                        vals[j * kNpw + q] = lam * dtx;
                        vals[kBT * kNpw + j * kNpw + q] = gg * hs[j][q];
                    }
                    // sum_n lam dt B = dt lb; sum_n lam (A Abar h_{t-1} + B x) = dap + x lb
                    lds.slot[pl.w][j][lane] = dt * lb;
                    lds.slot[pl.w][j][kWave + lane] = fmaf(x, lb, dap);
                    lds.slot[pl.w][j][2 * kWave + lane] = pp;
                } else {
#pragma unroll
                    for (int q = 0; q < kNpw; ++q) {
                        vals[j * kNpw + q] = 0.0f;
                        vals[kBT * kNpw + j * kNpw + q] = 0.0f;
                    }
                }
              }
            }

            // dB, dC of this tile summed over the group's channels
            {
                const float sum = lane_sums(vals);
                const int v = reverse6(lane);
                const int which = v / (kBT * kNpw);
                const int r = v - which * kBT * kNpw;
                const int j = r / kNpw;
                const int n = pl.n0 + (r - j * kNpw);
                if (j < cnt && n < N) {
                    part_bc[(which * ws.nslots + pl.grp) * bc_slot_floats(f) + bc_index(f, pl.b, t0 + j, n)] =
                        sum;
                }
            }
            __syncthreads();

            // finish this wave's tokens of the tile
#pragma unroll
            for (int jj = 0; jj < OW; ++jj) {
                const int j = jj * S + pl.w;
                if (j < cnt) {
                    float dxs = 0.0f, dds = 0.0f, ps = 0.0f;
#pragma unroll
                    for (int u = 0; u < S; ++u) {
                        dxs += lds.slot[u][j][lane];
                        dds += lds.slot[u][j][kWave + lane];
                        ps += lds.slot[u][j][2 * kWave + lane];
                    }
                    const Own o = own[jj];
                    const float gg = lds.g[j][lane];
                    if constexpr (HAS_D) {
                        dxs = fmaf(dskip, gg, dxs);
                        ps = fmaf(dskip, o.x, ps);
                    }
                    const float dv = SP ? dds * sigmoid_f32(o.v) : dds;
                    dD_acc = fmaf(gg, o.x, dD_acc);
                    dbias_acc += dv;
                    if (pl.valid) {
                        const int64_t idx = (pl.b * L + t0 + j) * f.dim + pl.d;
                        store_io<IO>(a.dx, idx, dxs);
                        store_io<IO>(a.ddelta, idx, dv);
                        if constexpr (HAS_Z) {
                            const float s = sigmoid_f32(o.z);
                            store_io<IO>(a.dz, idx, o.dy * ps * (s * fmaf(o.z, 1.0f - s, 1.0f)));
                        }
                    }
                }
            }
        }
    }

    // the gradient at h0 (first chunk; later chunks' Abar lam is what their
    // left neighbour takes in, already folded by the carry) and the
    // per-(chunk, row) partials of dA, dD, d bias
    if constexpr (MODE != kBwdForward) {
        const int64_t prow = chunk * f.batch + pl.b;
        if (pl.valid) {
#pragma unroll
            for (int q = 0; q < kNpw; ++q) {
                if (sv[q]) {
                    const int64_t col = (pl.b * f.dim + pl.d) * N + pl.n0 + q;
                    if (chunk == 0 && a.dh0 != nullptr) a.dh0[col] = m[q];
                    part_a[(prow * f.dim + pl.d) * N + pl.n0 + q] = dA[q];
                }
            }
        }
        __syncthreads();
        lds.slot[pl.w][0][lane] = dD_acc;
        lds.slot[pl.w][0][kWave + lane] = dbias_acc;
        __syncthreads();
        if (pl.w == 0 && pl.valid) {
            float sd = 0.0f, sb = 0.0f;
#pragma unroll
            for (int u = 0; u < S; ++u) {
                sd += lds.slot[u][0][lane];
                sb += lds.slot[u][0][kWave + lane];
            }
            part_d[prow * f.dim + pl.d] = sd;
            part_bias[prow * f.dim + pl.d] = sb;
        }
    }
}

// ---------------------------------------------------------------------------
// A sequence cut into chunks, for shapes whose channel groups alone do not
// fill the chip. Each (chunk, row, group) workgroup of the main kernel walks
// only its chunk and needs the state entering it and the adjoint entering it
// from the right. Both are first-order linear recurrences over the chunks:
// the state after chunk c is P_c h + e_c with e_c the chunk's end state from
// a zero start and P_c = exp(A * sum of delta over the chunk); the adjoint
// the chunk hands to its left neighbour, Abar of its first token times lam
// there, is P_c rho + l_c with rho what it takes in and l_c the same walked
// back from zero. Each chunk is summarised, and the summaries are folded in
// order (forward for the states, from the last chunk back for the adjoint).
// The state summaries come from the forward pass itself: it runs every chunk
// from a zero state, so its checkpoints lack the entering state h, which at
// the checkpoint of tile i has decayed to exp(A * s_i) h, s_i the sum of
// delta over the chunk before the tile; the walk back, launched after the
// folds, adds that term to each checkpoint it reads.

// Adjoint summary of chunks 1 .. nchunks-1, walked back from a zero adjoint
// (the last chunk from dhL): what the chunk hands to its left neighbour and
// its decay product, stored at [nchunks - 1 - chunk][b][d][n] so that the
// same in-order fold gives the adjoints.
template <int S, int IO, bool SP, bool HAS_Z>
__device__ __forceinline__ void bwd_adjoint_summary(const BwdArgs& a, int64_t ngroups,
                                                    const BwdWs& ws, float* end, float* decay,
                                                    int64_t blk, BwdLdsIn<S>& lds) {
    const ScanArgs& f = a.fwd;
    const int N = f.dstate;
    const int64_t L = f.seqlen;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t rows = f.batch * ngroups;
    const int64_t chunk = 1 + blk / rows;
    const Place pl = make_place(f, ngroups, blk - (chunk - 1) * rows);
    const bool last_chunk = chunk == ws.nchunks - 1;
    const int64_t i_first = chunk * (ws.chunk_len / kBT);
    const int64_t i_end = last_chunk ? (L + kBT - 1) / kBT : i_first + ws.chunk_len / kBT;
    const int64_t col0 = (pl.b * f.dim + pl.d) * N;
    bool sv[kNpw];
    float A2[kNpw], lam[kNpw], en[kNpw];
#pragma unroll
    for (int q = 0; q < kNpw; ++q) {
        const int n = pl.n0 + q;
        sv[q] = n < N;
        A2[q] = sv[q] ? f.A[pl.d * N + n] * kLog2e : 0.0f;
        lam[q] = (last_chunk && sv[q] && a.dhL != nullptr) ? a.dhL[col0 + n] : 0.0f;
        en[q] = 1.0f;
    }
    float dsum = 0.0f;
    Own own[(kBT + S - 1) / S];
    // tiles fetched kAhead ahead, as in the forward pass (without the
    // checkpoints, which the summary does not read)
    TileRaw<S> raw[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
        const int64_t pv = max(i_end - 1 - u, i_first);
        fetch_tile<S, IO, HAS_Z, true, false, false>(
            a, pl, ws.tent, pv, static_cast<int>(min<int64_t>(kBT, L - pv * kBT)), raw[u]);
    }
    for (int64_t i0 = i_end - 1; i0 >= i_first; i0 -= kAhead) {
#pragma unroll
        for (int u = 0; u < kAhead; ++u) {
            const int64_t i = i0 - u;
            if (i < i_first) break;
            // tokens past the end of the sequence are staged inert (g = delta
            // = 0, zero C rows): they leave lam, en and the sum unchanged
            put_tile<S, IO, SP, HAS_Z, true>(raw[u], pl, lds,
                                             static_cast<int>(min<int64_t>(kBT, L - i * kBT)), N, own);
            __syncthreads();
            {
                // the first tiles fetch the first one again (unused)
                const int64_t pv = max(i - kAhead, i_first);
                fetch_tile<S, IO, HAS_Z, true, false, false>(
                    a, pl, ws.tent, pv, static_cast<int>(min<int64_t>(kBT, L - pv * kBT)), raw[u]);
            }
#pragma unroll
            for (int j1 = kBT - 1; j1 >= 0; j1 -= 2) {
                float2 vv[2];
                float gq[2];
                f32x4 cq[2];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    vv[jj] = lds.dtx[j1 - jj][lane];
                    gq[jj] = lds.g[j1 - jj][lane];
                    cq[jj] = *reinterpret_cast<const f32x4*>(&lds.bc[1][j1 - jj][pl.n0]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    dsum += vv[jj].x;
#pragma unroll
                    for (int q = 0; q < kNpw; ++q) {
                        lam[q] = fmaf(en[q], lam[q], cq[jj][q] * gq[jj]);
                        en[q] = fast_exp2(vv[jj].x * A2[q]);
                    }
                }
            }
            __syncthreads();
        }
    }
    if (pl.valid) {
        const int64_t at = (ws.nchunks - 1 - chunk) * f.batch * f.dim * N + col0 + pl.n0;
#pragma unroll
        for (int q = 0; q < kNpw; ++q) {
            if (sv[q]) {
                end[at + q] = en[q] * lam[q];
                decay[at + q] = fast_exp2(A2[q] * dsum);
            }
        }
    }
}

struct BwdCarry {
    float *fend, *fdecay, *fstart, *rend, *rdecay, *rstart;
};

// One thread per (b, d, n) column folds the summaries in order: start[k] =
// what enters summary k, k = 1 .. nchunks-1 (entry 0 is the first one's own);
// threads [0, columns) fold the states, [columns, 2 columns) the adjoints.
__global__ __launch_bounds__(256) void bwd_fold_kernel(int64_t columns, int64_t nchunks,
                                                       BwdCarry c) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
         t < 2 * columns; t += stride) {
        const bool adj = t >= columns;
        const int64_t col = adj ? t - columns : t;
        const float* end = adj ? c.rend : c.fend;
        const float* decay = adj ? c.rdecay : c.fdecay;
        float* start = adj ? c.rstart : c.fstart;
        float H = end[col];
        for (int64_t k = 1; k < nchunks; ++k) {
            start[k * columns + col] = H;
            if (k < nchunks - 1) H = fmaf(decay[k * columns + col], H, end[k * columns + col]);
        }
    }
}

// ---------------------------------------------------------------------------
// Half channel groups (dstate 13..16, 4 waves). As in the forward scan, a
// launch of G groups on C compute units leaves some units a workgroup more
// than others unless C divides G, and the plan can run the last groups as
// two halves of 32 channels: lanes 0..31 and 32..63 of wave w take state
// split v = 2w and 2w + 1 of 8 (2 states each, padded past dstate) for the
// same 32 channels, so a lane does half a whole lane's state work. Split v
// also stages and finishes token v of every 8-token tile. Per-token sums over
// states go through LDS as 8 partials, and dB, dC are summed over the 32
// channels of each half-wave row by lane_sums32; a group's second half
// writes them to its own slot, which the reduction adds for split groups.
constexpr int kHalfCh = kHalfChannels;
constexpr int kHalfNps = 16 / kHalfSplits;  // states per lane of a half group
constexpr int kHalfVals = 2 * kBT * kHalfNps;
static_assert(kHalfVals == kWave / 2, "the half butterfly leaves one sum per lane");

struct BwdHalfLds {
    float2 dtx[kBT][kHalfCh];
    float g[kBT][kHalfCh];
    alignas(16) float bc[2][kBT][kHalfSplits * kHalfNps];
    float red[3][kHalfSplits][kBT][kHalfCh];
};

template <int IO, bool SP, bool HAS_D, bool HAS_Z>
__device__ __forceinline__ void bwd_half_group(const BwdArgs& a, int64_t ngroups, int64_t b,
                                               int64_t grp, int side, const BwdWs& ws,
                                               BwdHalfLds& lds) {
    constexpr int NP = kHalfSplits * kHalfNps;  // 16 padded states
    const ScanArgs& f = a.fwd;
    const int N = f.dstate;
    const int64_t L = f.seqlen;
    const int lane = threadIdx.x & (kWave - 1);
    const int ch = lane & (kHalfCh - 1);
    const int v = 2 * (static_cast<int>(threadIdx.x) / kWave) + (lane >> 5);
    const int n0 = v * kHalfNps;
    const int64_t d_raw = grp * kWave + side * kHalfCh + ch;
    const bool valid = d_raw < f.dim;
    const int64_t d = valid ? d_raw : f.dim - 1;
    const float dbias = f.delta_bias != nullptr ? f.delta_bias[d] : 0.0f;
    const float dskip = HAS_D ? f.D[d] : 0.0f;
    const int64_t slot = side == 0 ? grp : ngroups + grp;

    bool sv[kHalfNps];
    // m: Abar lam of the token after the one being walked, dhL at the end
    float A[kHalfNps], A2[kHalfNps], m[kHalfNps], dA[kHalfNps];
#pragma unroll
    for (int q = 0; q < kHalfNps; ++q) {
        const int n = n0 + q;
        sv[q] = n < N;
        A[q] = sv[q] ? f.A[d * N + n] : 0.0f;
        A2[q] = A[q] * kLog2e;
        m[q] = (sv[q] && a.dhL != nullptr) ? a.dhL[(b * f.dim + d) * N + n] : 0.0f;
        dA[q] = 0.0f;
    }
    float dD_acc = 0.0f, dbias_acc = 0.0f;
    Own own;

    struct Raw {
        uint32_t x, dl, dy, z, bc;
        float he[kHalfNps];
    };
    // token v of tile `tile` for this lane's channel, one B or C element per
    // thread and, walking backwards, the tile's checkpointed states; every
    // index clamped into range (the clamped values are never used)
    auto fetch = [&](auto want_g, int64_t tile, int cnt, Raw& r) {
        constexpr bool WANT_G = decltype(want_g)::value;
        const int64_t t0 = tile * kBT;
        const int j = min(v, cnt - 1);
        const int64_t idx = (b * L + t0 + j) * f.dim + d;
        r.x = load_raw<IO>(f.x, idx);
        r.dl = load_raw<IO>(f.delta, idx);
        if constexpr (WANT_G) {
            r.dy = load_raw<IO>(a.dy, idx);
            r.z = HAS_Z ? load_raw<IO>(f.z, idx) : 0u;
        }
        const int e = threadIdx.x;  // exactly one B or C element per thread
        const int which = e / (kBT * NP);
        const int rr = e - which * kBT * NP;
        const int jb = min(rr / NP, cnt - 1);
        const int n = min(rr % NP, N - 1);
        r.bc = load_raw<IO>(which ? f.C : f.B, (b * L + t0 + jb) * N + n);
        if constexpr (WANT_G) {
            const float2 v = *reinterpret_cast<const float2*>(ws.tent + tent_index(f, tile, b, d, n0));
            r.he[0] = v.x;
            r.he[1] = v.y;
        }
    };
    auto put = [&](auto want_g, const Raw& r, int cnt) {
        constexpr bool WANT_G = decltype(want_g)::value;
        if (v < cnt) {
            float xf = raw_to_f32<IO>(r.x);
            const float vv = raw_to_f32<IO>(r.dl) + dbias;
            const float dt = SP ? softplus_f32(vv) : vv;
            if (!valid) xf = 0.0f;  // a clamped lane contributes nothing
            lds.dtx[v][ch] = make_float2(dt, xf);
            if constexpr (WANT_G) {
                const float dyf = raw_to_f32<IO>(r.dy);
                const float zf = HAS_Z ? raw_to_f32<IO>(r.z) : 0.0f;
                float gg = HAS_Z ? dyf * silu(zf) : dyf;
                if (!valid) gg = 0.0f;
                lds.g[v][ch] = gg;
                own = Own{dyf, zf, vv, xf};
            }
        } else {
            // past the end of the sequence: inert, as in whole groups
            lds.dtx[v][ch] = make_float2(0.0f, 0.0f);
            if constexpr (WANT_G) lds.g[v][ch] = 0.0f;
        }
        const int e = threadIdx.x;
        const int which = e / (kBT * NP);
        const int rr = e - which * kBT * NP;
        const bool in = rr / NP < cnt && rr % NP < N;  // padding states and tokens read as 0
        lds.bc[which][rr / NP][rr % NP] = in ? raw_to_f32<IO>(r.bc) : 0.0f;
    };
    using No = std::integral_constant<bool, false>;
    using Yes = std::integral_constant<bool, true>;

    const int64_t ntiles = (L + kBT - 1) / kBT;
    // (1) forward over the whole sequence, keeping the state entering every
    // tile (only real lanes and states write)
    {
        float h[kHalfNps];
#pragma unroll
        for (int q = 0; q < kHalfNps; ++q)
            h[q] = (sv[q] && f.h0 != nullptr) ? f.h0[(b * f.dim + d) * N + n0 + q] : 0.0f;
        Raw raw;
        fetch(No{}, 0, static_cast<int>(min<int64_t>(kBT, L)), raw);
        set_prio(3);
        for (int64_t i = 0; i < ntiles; ++i) {
            const int64_t t0 = i * kBT;
            const int cnt = static_cast<int>(min<int64_t>(kBT, L - t0));
            if (valid)   // padding states hold zero
                *reinterpret_cast<float2*>(ws.tent + tent_index(f, i, b, d, n0)) = make_float2(h[0], h[1]);
            put(No{}, raw, cnt);
            __syncthreads();
            {
                const int64_t nx = min(i + 1, ntiles - 1);
                fetch(No{}, nx, static_cast<int>(min<int64_t>(kBT, L - nx * kBT)), raw);
            }
#pragma unroll
            for (int j0 = 0; j0 < kBT; j0 += 2) {
                float2 vq[2], bq[2];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    vq[jj] = lds.dtx[j0 + jj][ch];
                    bq[jj] = *reinterpret_cast<const float2*>(&lds.bc[0][j0 + jj][n0]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const float du = vq[jj].x * vq[jj].y;
                    h[0] = fmaf(fast_exp2(vq[jj].x * A2[0]), h[0], du * bq[jj].x);
                    h[1] = fmaf(fast_exp2(vq[jj].x * A2[1]), h[1], du * bq[jj].y);
                }
            }
            __syncthreads();
        }
    }

    // (2) the tiles in reverse
    {
        Raw raw;
        fetch(Yes{}, ntiles - 1, static_cast<int>(L - (ntiles - 1) * kBT), raw);
        const PrioSteps prio(ntiles, 2);
        for (int64_t i = ntiles - 1; i >= 0; --i) {
            prio.at(ntiles - 1 - i, 2);
            const int64_t t0 = i * kBT;
            const int cnt = static_cast<int>(min<int64_t>(kBT, L - t0));
            // the recomputed states and the decay factors of the tile's
            // tokens stay in registers for the walk back (2 states per lane)
            float he[kHalfNps], hs[kBT][kHalfNps], ev[kBT][kHalfNps], h[kHalfNps];
#pragma unroll
            for (int q = 0; q < kHalfNps; ++q) he[q] = (valid && sv[q]) ? raw.he[q] : 0.0f;
            put(Yes{}, raw, cnt);
            __syncthreads();
            fetch(Yes{}, i > 0 ? i - 1 : 0, kBT < L ? kBT : static_cast<int>(L), raw);

#pragma unroll
            for (int q = 0; q < kHalfNps; ++q) h[q] = he[q];
#pragma unroll
            for (int j0 = 0; j0 < kBT; j0 += 2) {
                float2 vq[2], bq[2];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    vq[jj] = lds.dtx[j0 + jj][ch];
                    bq[jj] = *reinterpret_cast<const float2*>(&lds.bc[0][j0 + jj][n0]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int j = j0 + jj;
                    const float du = vq[jj].x * vq[jj].y;
                    ev[j][0] = fast_exp2(vq[jj].x * A2[0]);
                    ev[j][1] = fast_exp2(vq[jj].x * A2[1]);
                    h[0] = fmaf(ev[j][0], h[0], du * bq[jj].x);
                    h[1] = fmaf(ev[j][1], h[1], du * bq[jj].y);
                    hs[j][0] = h[0];
                    hs[j][1] = h[1];
                }
            }

            // dB and dC terms: set token by token (zero past the sequence)
            float vals[kHalfVals];
#pragma unroll
            for (int j1 = kBT - 1; j1 >= 0; j1 -= 2) {
                float2 vv[2], bq[2], cq[2];
                float gq[2];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    vv[jj] = lds.dtx[j1 - jj][ch];
                    gq[jj] = lds.g[j1 - jj][ch];
                    bq[jj] = *reinterpret_cast<const float2*>(&lds.bc[0][j1 - jj][n0]);
                    cq[jj] = *reinterpret_cast<const float2*>(&lds.bc[1][j1 - jj][n0]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int j = j1 - jj;
                    if (j < cnt) {
                        const float dt = vv[jj].x, x = vv[jj].y;
                        const float gg = gq[jj];
                        const float Bv[kHalfNps] = {bq[jj].x, bq[jj].y};
                        const float Cv[kHalfNps] = {cq[jj].x, cq[jj].y};
                        const float dtx = dt * x;
                        float lb = 0.0f, dap = 0.0f, pp = 0.0f;
#pragma unroll
                        for (int q = 0; q < kHalfNps; ++q) {
                            const float lam = fmaf(Cv[q], gg, m[q]);
                            const float hprev = j > 0 ? hs[j > 0 ? j - 1 : 0][q] : he[q];
                            m[q] = ev[j][q] * lam;
                            const float le = m[q] * hprev;
                            dA[q] = fmaf(dt, le, dA[q]);
                            dap = fmaf(A[q], le, dap);
                            lb = fmaf(lam, Bv[q], lb);
                            pp = fmaf(Cv[q], hs[j][q], pp);
                            vals[j * kHalfNps + q] = lam * dtx;
                            vals[kBT * kHalfNps + j * kHalfNps + q] = gg * hs[j][q];
                        }
                        lds.red[0][v][j][ch] = dt * lb;
                        lds.red[1][v][j][ch] = fmaf(x, lb, dap);
                        lds.red[2][v][j][ch] = pp;
                    } else {
#pragma unroll
                        for (int q = 0; q < kHalfNps; ++q) {
                            vals[j * kHalfNps + q] = 0.0f;
                            vals[kBT * kHalfNps + j * kHalfNps + q] = 0.0f;
                        }
                    }
                }
            }

            // dB, dC of this tile summed over the half's 32 channels
            {
                const float sum = lane_sums32(vals);
                const int r5 = reverse5(ch);
                const int which = r5 / (kBT * kHalfNps);
                const int r = r5 - which * kBT * kHalfNps;
                const int j = r / kHalfNps;
                const int n = n0 + (r - j * kHalfNps);
                if (j < cnt && n < N) {
                    ws.part_bc[(which * ws.nslots + slot) * bc_slot_floats(f) + bc_index(f, b, t0 + j, n)] =
                        sum;
                }
            }
            __syncthreads();

            // finish this lane's token v of the tile: the 8 split partials
            if (v < cnt) {
                float dxs = 0.0f, dds = 0.0f, ps = 0.0f;
#pragma unroll
                for (int u = 0; u < kHalfSplits; ++u) {
                    dxs += lds.red[0][u][v][ch];
                    dds += lds.red[1][u][v][ch];
                    ps += lds.red[2][u][v][ch];
                }
                const float gg = lds.g[v][ch];
                if constexpr (HAS_D) {
                    dxs = fmaf(dskip, gg, dxs);
                    ps = fmaf(dskip, own.x, ps);
                }
                const float dv = SP ? dds * sigmoid_f32(own.v) : dds;
                dD_acc = fmaf(gg, own.x, dD_acc);
                dbias_acc += dv;
                if (valid) {
                    const int64_t idx = (b * L + t0 + v) * f.dim + d;
                    store_io<IO>(a.dx, idx, dxs);
                    store_io<IO>(a.ddelta, idx, dv);
                    if constexpr (HAS_Z) {
                        const float sg = sigmoid_f32(own.z);
                        store_io<IO>(a.dz, idx, own.dy * ps * (sg * fmaf(own.z, 1.0f - sg, 1.0f)));
                    }
                }
            }
        }
    }

    // gradients at h0 and the per-row partials of dA, dD, d bias
    if (valid) {
#pragma unroll
        for (int q = 0; q < kHalfNps; ++q) {
            if (sv[q]) {
                const int64_t col = (b * f.dim + d) * N + n0 + q;
                if (a.dh0 != nullptr) a.dh0[col] = m[q];
                ws.part_a[col] = dA[q];
            }
        }
    }
    __syncthreads();
    lds.red[0][v][0][ch] = dD_acc;
    lds.red[1][v][0][ch] = dbias_acc;
    __syncthreads();
    if (v == 0 && valid) {
        float sd = 0.0f, sb = 0.0f;
#pragma unroll
        for (int u = 0; u < kHalfSplits; ++u) {
            sd += lds.red[0][u][0][ch];
            sb += lds.red[1][u][0][ch];
        }
        ws.part_d[b * f.dim + d] = sd;
        ws.part_bias[b * f.dim + d] = sb;
    }
}

// One launch of whole and half groups (dstate 13..16): blocks [0, nwhole)
// are whole groups in (row, group) order, the blocks after them the two
// halves of each remaining group, placed by half_block_pair.
template <int IO, bool SP, bool HAS_D, bool HAS_Z>
__global__ __launch_bounds__(kWave * 4) __attribute__((amdgpu_waves_per_eu(3)))
void scan_bwd_mixed_kernel(BwdArgs a, int64_t ngroups, int64_t nwhole, BwdWs ws) {
    __shared__ union {
        BwdLds<4> whole;
        BwdHalfLds half;
    } lds;
    const int64_t blk = blockIdx.x;
    if (blk < nwhole) {
        bwd_whole_group<4, IO, SP, HAS_D, HAS_Z>(a, ngroups, blk, ws, lds.whole);
    } else {
        int64_t pair;
        int side;
        half_block_pair(blk - nwhole, static_cast<int64_t>(gridDim.x) - nwhole, pair, side);
        const int64_t gi = nwhole + pair;  // (row, group) index of the split group
        bwd_half_group<IO, SP, HAS_D, HAS_Z>(a, ngroups, gi / ngroups, gi % ngroups, side, ws,
                                             lds.half);
    }
}

template <int S, int IO, bool SP, bool HAS_D, bool HAS_Z, int MODE>
__global__ __launch_bounds__(kWave * S) __attribute__((amdgpu_waves_per_eu(S == 4 ? 3 : 1)))
void scan_bwd_kernel(BwdArgs a, int64_t ngroups, BwdWs ws) {
    __shared__ BwdLds<S> lds;
    bwd_whole_group<S, IO, SP, HAS_D, HAS_Z, MODE>(a, ngroups, blockIdx.x, ws, lds);
}

// A chunked sequence, first launch: blocks [0, nfwd) run the forward pass of
// every (chunk, row, group) from a zero state (chunk 0 from h0), writing the
// checkpoints, the tiles' delta sums and the chunk summaries of the states;
// the blocks after them summarise the adjoints of chunks 1 .. nchunks-1.
// Both are independent of the carries, which are folded after this launch.
template <int S, int IO, bool SP, bool HAS_Z>
__global__ __launch_bounds__(kWave * S) void bwd_forward_kernel(BwdArgs a, int64_t ngroups,
                                                                BwdWs ws, BwdCarry c,
                                                                int64_t nfwd) {
    __shared__ BwdLdsIn<S> lds;
    const int64_t blk = blockIdx.x;
    if (blk < nfwd)
        bwd_whole_group<S, IO, SP, false, false, kBwdForward>(a, ngroups, blk, ws, lds);
    else
        bwd_adjoint_summary<S, IO, SP, HAS_Z>(a, ngroups, ws, c.rend, c.rdecay, blk - nfwd, lds);
}

// dB and dC: the partials of all channel groups added in group order, a
// split group's second half right after its first. Groups of row b from
// index nwhole on in (row, group) order are split. Threads walk the
// partials' layout (per floats per slot, [row][group of 4 states][token][4])
// so their loads are contiguous; padding states are skipped.
__global__ __launch_bounds__(256) void bwd_bc_reduce_kernel(int64_t per, int64_t seqlen,
                                                            int dstate, int64_t ngroups,
                                                            int64_t nslots, int64_t nwhole,
                                                            const float* part, float* dB,
                                                            float* dC) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t row = ((dstate + 3) / 4) * seqlen * 4;   // floats of one batch row
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < 2 * per;
         i += stride) {
        const int64_t which = i / per;
        const int64_t r = i - which * per;
        const int64_t b = r / row;
        const int64_t gq = r - b * row;
        const int64_t grp4 = gq / (seqlen * 4);
        const int64_t tq = gq - grp4 * seqlen * 4;
        const int64_t t = tq >> 2;
        const int n = static_cast<int>(grp4 * 4 + (tq & 3));
        if (n >= dstate) continue;
        const int64_t first_split = nwhole - b * ngroups;  // groups of this row
        const bool halves = first_split < ngroups;
        // 8 groups' partials are loaded before they are added (in group order),
        // so a thread waits for memory once per 8 groups
        float s = 0.0f;
        for (int64_t g0 = 0; g0 < ngroups; g0 += 8) {
            float p[8], e[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t g = min(g0 + u, ngroups - 1);  // clamped, the copy is unused
                p[u] = part[(which * nslots + g) * per + r];
                e[u] = halves ? part[(which * nslots + ngroups + g) * per + r] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t g = g0 + u;
                if (g < ngroups) {
                    s += p[u];
                    if (g >= first_split) s += e[u];  // only split groups' second halves
                }
            }
        }
        (which ? dC : dB)[(b * seqlen + t) * dstate + n] = s;
    }
}

// dA, dD, d bias: the per-row partials (rows: chunks x batch rows) added in
// row order, loading kParamBatch rows before adding them so a thread waits
// for memory once per batch of rows.
constexpr int kParamBatch = 8;

__global__ __launch_bounds__(256) void bwd_param_reduce_kernel(int64_t rows, int64_t dim, int N,
                                                               const float* part_a,
                                                               const float* part_d,
                                                               const float* part_bias, float* dA,
                                                               float* dD, float* dbias) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t cols = dim * N;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < cols;
         i += stride) {
        float s = 0.0f;
        for (int64_t b0 = 0; b0 < rows; b0 += kParamBatch) {
            float v[kParamBatch];
#pragma unroll
            for (int u = 0; u < kParamBatch; ++u)
                v[u] = part_a[min(b0 + u, rows - 1) * cols + i];  // clamped: unused past rows
#pragma unroll
            for (int u = 0; u < kParamBatch; ++u)
                if (b0 + u < rows) s += v[u];
        }
        dA[i] = s;
        if (i < dim) {
            float sd = 0.0f, sb = 0.0f;
            for (int64_t b0 = 0; b0 < rows; b0 += kParamBatch) {
                float vd[kParamBatch], vb[kParamBatch];
#pragma unroll
                for (int u = 0; u < kParamBatch; ++u) {
                    const int64_t b = min(b0 + u, rows - 1);
                    vd[u] = part_d[b * dim + i];
                    vb[u] = part_bias[b * dim + i];
                }
#pragma unroll
                for (int u = 0; u < kParamBatch; ++u) {
                    if (b0 + u < rows) {
                        sd += vd[u];
                        sb += vb[u];
                    }
                }
            }
            if (dD != nullptr) dD[i] = sd;
            if (dbias != nullptr) dbias[i] = sb;
        }
    }
}

// Empty sequence or empty batch: dA, dD, d bias are zero and dh0 = dhL.
__global__ __launch_bounds__(256) void bwd_degenerate_kernel(int64_t cols, int64_t dim,
                                                             int64_t states, const float* dhL,
                                                             float* dA, float* dD, float* dbias,
                                                             float* dh0) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t n = cols > states ? cols : states;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += stride) {
        if (i < cols) dA[i] = 0.0f;
        if (i < dim) {
            if (dD != nullptr) dD[i] = 0.0f;
            if (dbias != nullptr) dbias[i] = 0.0f;
        }
        if (i < states && dh0 != nullptr) dh0[i] = dhL != nullptr ? dhL[i] : 0.0f;
    }
}

struct BwdLayout {
    int64_t ntiles, ngroups, nslots, nchunks, chunk_len;
    size_t tent, part_bc, part_a, part_d, part_bias;          // float offsets
    size_t fend, fdecay, fstart, rend, rdecay, rstart;        // chunk carries (nchunks > 1)
    size_t dpre;                                              // [tile][b][d] (nchunks > 1)
    size_t total;                                             // float count
};

// Half groups need 4 waves of states (dstate 13..16).
inline bool bwd_halvable(int dstate) { return bwd_halves_supported(dstate); }
static_assert(kNpw * 4 == 16, "dstate 13..16 fills 4 waves");

inline size_t round64(size_t v) { return (v + 63) / 64 * 64; }

BwdLayout bwd_layout(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int64_t chunk_len) {
    BwdLayout l;
    l.ntiles = (seqlen + kBT - 1) / kBT;
    l.ngroups = (dim + kWave - 1) / kWave;
    l.chunk_len = chunk_len > 0 ? chunk_len : l.ntiles * kBT;
    l.nchunks = chunk_len > 0 ? (seqlen + chunk_len - 1) / chunk_len : 1;
    // slots for the second halves of split groups whenever the shape allows
    // splitting, so the size needs no knowledge of the device; a chunked
    // plan never splits groups (halves need the whole sequence)
    l.nslots = bwd_halvable(dstate) && l.nchunks == 1 ? 2 * l.ngroups : l.ngroups;
    const size_t states = static_cast<size_t>(batch) * dim * dstate;
    size_t off = 0;
    l.tent = off;   // states padded to whole groups of 4
    off += round64(static_cast<size_t>(l.ntiles) * batch * dim * ((dstate + 3) / 4 * 4));
    l.part_bc = off;   // states padded to whole groups of 4
    off += round64(2 * static_cast<size_t>(l.nslots) * batch * seqlen * ((dstate + 3) / 4 * 4));
    const size_t nc = static_cast<size_t>(l.nchunks);
    l.part_a = off;
    off += round64(nc * states);
    l.part_d = off;
    off += round64(nc * batch * dim);
    l.part_bias = off;
    off += round64(nc * batch * dim);
    const size_t carry = l.nchunks > 1 ? round64(nc * states) : 0;
    l.fend = off;
    off += carry;
    l.fdecay = off;
    off += carry;
    l.fstart = off;
    off += carry;
    l.rend = off;
    off += carry;
    l.rdecay = off;
    off += carry;
    l.rstart = off;
    off += carry;
    l.dpre = off;
    off += l.nchunks > 1 ? round64(static_cast<size_t>(l.ntiles) * batch * dim) : 0;
    l.total = off;
    return l;
}

template <int S, int IO, bool SP>
hipError_t launch_bwd_main(const BwdArgs& a, const BwdLayout& l, float* ws, hipStream_t s) {
    const int64_t groups = a.fwd.batch * l.ngroups;
    const bool has_d = a.fwd.D != nullptr, has_z = a.fwd.z != nullptr;
    const BwdWs w{ws + l.tent, ws + l.part_bc, ws + l.part_a, ws + l.part_d, ws + l.part_bias,
                  l.nslots, l.nchunks, l.chunk_len, ws + l.fstart, ws + l.rstart,
                  ws + l.fend, ws + l.fdecay, ws + l.dpre};
    if constexpr (S == 4) {
        if (a.halves > 0) {
            const int64_t nwhole = groups - a.halves;
            const dim3 grid(nwhole + 2 * a.halves), block(kWave * S);
            auto go = [&](auto kernel) {
                hipLaunchKernelGGL(kernel, grid, block, 0, s, a, l.ngroups, nwhole, w);
            };
            if (has_d && has_z) go(scan_bwd_mixed_kernel<IO, SP, true, true>);
            else if (has_d) go(scan_bwd_mixed_kernel<IO, SP, true, false>);
            else if (has_z) go(scan_bwd_mixed_kernel<IO, SP, false, true>);
            else go(scan_bwd_mixed_kernel<IO, SP, false, false>);
            return hipGetLastError();
        }
    }
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(l.nchunks * groups), dim3(kWave * S), 0, s, a, l.ngroups,
                           w);
    };
    if (l.nchunks == 1) {
        if (has_d && has_z) go(scan_bwd_kernel<S, IO, SP, true, true, kBwdBoth>);
        else if (has_d) go(scan_bwd_kernel<S, IO, SP, true, false, kBwdBoth>);
        else if (has_z) go(scan_bwd_kernel<S, IO, SP, false, true, kBwdBoth>);
        else go(scan_bwd_kernel<S, IO, SP, false, false, kBwdBoth>);
        return hipGetLastError();
    }
    // a chunked sequence: the forward pass of every chunk from a zero state
    // and the adjoint summaries, the two folds (states forward, adjoints
    // backward), then the walk back of every chunk, which adds the folded
    // entering state to its checkpoints
    const int64_t columns = a.fwd.batch * a.fwd.dim * a.fwd.dstate;
    const int64_t nfwd = l.nchunks * groups;
    const int64_t nadj = (l.nchunks - 1) * groups;
    const BwdCarry c{ws + l.fend, ws + l.fdecay, ws + l.fstart,
                     ws + l.rend, ws + l.rdecay, ws + l.rstart};
    const dim3 grid(nfwd + nadj), block(kWave * S);
    if (has_z)
        hipLaunchKernelGGL((bwd_forward_kernel<S, IO, SP, true>), grid, block, 0, s, a, l.ngroups,
                           w, c, nfwd);
    else
        hipLaunchKernelGGL((bwd_forward_kernel<S, IO, SP, false>), grid, block, 0, s, a, l.ngroups,
                           w, c, nfwd);
    hipLaunchKernelGGL(bwd_fold_kernel, dim3(stride_blocks(2 * columns)), dim3(256), 0, s, columns,
                       l.nchunks, c);
    if (has_d && has_z) go(scan_bwd_kernel<S, IO, SP, true, true, kBwdWalk>);
    else if (has_d) go(scan_bwd_kernel<S, IO, SP, true, false, kBwdWalk>);
    else if (has_z) go(scan_bwd_kernel<S, IO, SP, false, true, kBwdWalk>);
    else go(scan_bwd_kernel<S, IO, SP, false, false, kBwdWalk>);
    return hipGetLastError();
}

template <int IO, bool SP>
hipError_t launch_bwd_io(const BwdArgs& a, float* ws, hipStream_t s) {
    const ScanArgs& f = a.fwd;
    const BwdLayout l = bwd_layout(f.batch, f.seqlen, f.dim, f.dstate, a.chunk_len);
    hipError_t e;
    switch ((f.dstate + kNpw - 1) / kNpw) {
        case 1: e = launch_bwd_main<1, IO, SP>(a, l, ws, s); break;
        case 2: e = launch_bwd_main<2, IO, SP>(a, l, ws, s); break;
        case 3: e = launch_bwd_main<3, IO, SP>(a, l, ws, s); break;
        case 4: e = launch_bwd_main<4, IO, SP>(a, l, ws, s); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int64_t per = f.batch * f.seqlen * ((f.dstate + 3) / 4 * 4);
    const int64_t nwhole = f.batch * l.ngroups - (bwd_halvable(f.dstate) ? a.halves : 0);
    hipLaunchKernelGGL(bwd_bc_reduce_kernel, dim3(stride_blocks(2 * per)), dim3(256), 0, s, per,
                       f.seqlen, f.dstate, l.ngroups, l.nslots, nwhole, ws + l.part_bc, a.dB, a.dC);
    hipLaunchKernelGGL(bwd_param_reduce_kernel, dim3(stride_blocks(f.dim * f.dstate)), dim3(256),
                       0, s, l.nchunks * f.batch, f.dim, f.dstate, ws + l.part_a, ws + l.part_d,
                       ws + l.part_bias, a.dA, a.dD, a.ddelta_bias);
    return hipGetLastError();
}

}  // namespace

size_t scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int dstate,
                                int64_t chunk_len) {
    if (batch == 0 || seqlen == 0 || dim == 0) return 0;
    return bwd_layout(batch, seqlen, dim, dstate, chunk_len).total * sizeof(float);
}

hipError_t launch_scan_bwd(const BwdArgs& a, void* workspace, hipStream_t stream) {
    const ScanArgs& f = a.fwd;
    if (f.dim == 0) return hipSuccess;
    if (f.batch == 0 || f.seqlen == 0) {
        const int64_t cols = f.dim * f.dstate;
        const int64_t states = f.batch * f.dim * f.dstate;
        hipLaunchKernelGGL(bwd_degenerate_kernel,
                           dim3(stride_blocks(cols > states ? cols : states)), dim3(256), 0,
                           stream, cols, f.dim, states, a.dhL, a.dA, a.dD, a.ddelta_bias, a.dh0);
        return hipGetLastError();
    }
    float* ws = static_cast<float*>(workspace);
    const bool sp = f.delta_softplus != 0;
    if (f.io == kIoF32)
        return sp ? launch_bwd_io<kIoF32, true>(a, ws, stream)
                  : launch_bwd_io<kIoF32, false>(a, ws, stream);
    return sp ? launch_bwd_io<kIoBF16, true>(a, ws, stream)
              : launch_bwd_io<kIoBF16, false>(a, ws, stream);
}

}  // namespace mamba
