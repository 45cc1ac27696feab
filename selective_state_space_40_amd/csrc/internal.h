// Internal interface between the C ABI layer (api.cpp, noalloc.hip) and the
// HIP kernels (scan_variant.hip, launch.hip, scan_bwd.hip, ssd.hip,
// conv1d.hip). Not installed; not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

struct mamba_scan_options;
struct mamba_scan_plan;

namespace mamba {

// Lanes of one wavefront on gfx950.
constexpr int kWave = 64;
// Channels covered by one workgroup of the scan kernels (one wave).
constexpr int kScanChannelsPerGroup = kWave;
// Tokens per register tile (the unit of prefetch and of the per-tile
// barrier); automatic chunk lengths are multiples of it.
#ifndef MAMBA_TOKEN_TILE
#define MAMBA_TOKEN_TILE 8
#endif
constexpr int kTokenTile = MAMBA_TOKEN_TILE;
// Tokens of a tile whose LDS inputs the scan reads together, ahead of their
// arithmetic (a divisor of kTokenTile).
constexpr int kLdsGroup = 2;

enum IoType : int { kIoF32 = 0, kIoBF16 = 1 };

// How one ssm_scan_fwd call is split: the sequence is cut into `nchunks`
// chunks of `chunk_len` tokens (the last one may be shorter).
// How chunks learn the state entering them (mamba_carry in the public
// header): a summary pass and a rerun of every chunk, or one pass from zero
// states and a rerun of each chunk's head only while the entering state
// still counts.
constexpr int kCarryRerun = 1;
constexpr int kCarryRepair = 2;

struct ScanPlan {
    int64_t chunk_len = 0;
    int64_t nchunks = 1;
    int state_split = 1;         // waves sharing the states of one channel
    int carry = kCarryRerun;     // kCarryRerun or kCarryRepair (nchunks > 1)
    int64_t halves = 0;          // last channel groups split into two 32-channel halves
    size_t workspace_bytes = 0;  // 0 when nchunks == 1
};

// State splits the kernels are built for: 1 for every dstate, and 2, 4, 8
// where they divide a dstate of 4, 8 or 16.
inline bool split_supported(int dstate, int split) {
    if (split == 1) return true;
    if (split != 2 && split != 4 && split != 8) return false;
    if (dstate != 4 && dstate != 8 && dstate != 16) return false;
    return dstate % split == 0;
}

struct ScanArgs {
    int64_t batch, seqlen, dim;
    int dstate;
    int io;
    const void* x;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* h0;
    void* y;
    float* hL;
    const float* delta_bias;  // (dim) or nullptr
    int delta_softplus;       // nonzero: delta <- softplus(delta + bias)
};

struct DecodeArgs {
    int64_t batch, dim;
    int dstate;
    int io;
    float* h;
    const void* x;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    void* y;
    const float* delta_bias;
    int delta_softplus;
};

// Widest short convolution the kernels are built for.
constexpr int kConvMaxWidth = 4;

// Short causal convolution. For the decode step seqlen is 1 and state_in
// and state_out are the same (batch, dim, width) buffer.
struct ConvArgs {
    int64_t batch, seqlen, dim;
    int width;
    int io;
    int silu;
    const void* x;
    const float* weight;
    const float* bias;
    const void* state_in;
    void* y;
    void* state_out;
    int fuse_state;  // set by the launcher: the forward kernel writes state_out itself
};

// Backward pass of the scan. The forward inputs come in `fwd` (its y and hL
// are not used); gradients of the loss sum(dy * y) + sum(dhL * hL).

struct BwdArgs {
    ScanArgs fwd;
    const void* dy;        // (batch, seqlen, dim) I/O dtype
    const float* dhL;      // (batch, dim, dstate) or nullptr
    void* dx;              // (batch, seqlen, dim) I/O dtype
    void* ddelta;          // (batch, seqlen, dim) I/O dtype: gradient at the delta input
    float* dA;             // (dim, dstate)
    float* dB;             // (batch, seqlen, dstate)
    float* dC;             // (batch, seqlen, dstate)
    float* dD;             // (dim) or nullptr
    void* dz;              // (batch, seqlen, dim) I/O dtype, or nullptr
    float* dh0;            // (batch, dim, dstate) or nullptr
    float* ddelta_bias;    // (dim) or nullptr
    int64_t halves = 0;    // last channel groups run as two 32-channel halves (dstate 13..16)
    int64_t chunk_len = 0; // tokens per chunk (a multiple of 8); 0: one chunk, no halves
};

// The backward pass can split channel groups into halves when a channel's
// states fill 4 waves of 4 (dstate 13..16).
inline bool bwd_halves_supported(int dstate) { return dstate >= 13 && dstate <= 16; }

// Scratch bytes of the backward pass for this shape cut into chunks of
// chunk_len tokens (0: one chunk).
size_t scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int dstate,
                                int64_t chunk_len);

// Queue the backward pass. Arguments are validated.
hipError_t launch_scan_bwd(const BwdArgs& a, void* workspace, hipStream_t stream);

// Mamba-2 dual form: heads of 64 channels sharing one decay and step.
struct SsdArgs {
    int64_t batch, seqlen, nheads;
    int dstate;            // 64 or 128
    const void* x;         // (batch, seqlen, nheads*64) bf16
    const void* dt;        // (batch, seqlen, nheads) bf16
    const float* A;        // (nheads)
    const void* B;         // (batch, seqlen, dstate) bf16
    const void* C;
    const float* D;        // (nheads*64) or nullptr
    const void* z;         // like x, or nullptr
    const float* h0;       // (batch, nheads, 64, dstate) or nullptr
    void* y;
    float* hL;
    const float* dt_bias;  // (nheads) or nullptr
    int dt_softplus;
};

hipError_t launch_ssd_fwd(const SsdArgs& a, hipStream_t stream);

// Workspace layout for nchunks > 1: three fp32 arrays of
// nchunks * batch * dim * dstate elements each: the state entering each
// chunk, each chunk's end state from a zero start, and each chunk's decay
// product.
size_t scan_workspace_bytes(int64_t batch, int64_t dim, int dstate, int64_t nchunks);

// Queue the kernels of one planned scan on `stream`. Arguments are already
// validated. Returns the HIP error of the last launch.
hipError_t launch_scan(const ScanArgs& a, const ScanPlan& plan, void* workspace,
                       hipStream_t stream);

// The chunked scan for one (I/O dtype, delta softplus) pair and half of the
// dstate range (PART 0: 1..8, PART 1: 9..16); each is compiled in its own
// translation unit (scan_variant.hip).
template <int IO, bool SP, int PART>
hipError_t launch_scan_variant(const ScanArgs& a, const ScanPlan& plan, void* workspace,
                               hipStream_t stream);

// Queue the convolution over whole sequences (update == false) or its
// decode step (update == true). Arguments are already validated.
hipError_t launch_conv1d(const ConvArgs& a, bool update, hipStream_t stream);

// Queue the single-token update. Arguments are already validated.
hipError_t launch_state_update(const DecodeArgs& a, hipStream_t stream);

// Where a forward scan without a workspace argument gets its scratch: asked
// for `bytes` once the plan is known (only when the plan needs scratch), it
// returns a mamba_status and sets *ws.
using ScratchSource = int (*)(size_t bytes, void** ws);

// ssm_scan_fwd's argument checks, plan and launch (api.cpp). With `scratch`
// non-null the workspace comes from it instead of the arguments.
int scan_fwd_call(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int dtype,
                  const void* x, const void* delta, const float* A, const void* B,
                  const void* C, const float* D, const void* z, const float* h0, void* y,
                  float* hL, const mamba_scan_options* options,
                  const mamba_scan_plan* plan_req, void* workspace, size_t workspace_bytes,
                  ScratchSource scratch, hipStream_t stream);

}  // namespace mamba
