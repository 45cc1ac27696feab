// Device helpers shared by the scan and decode kernels: I/O element access,
// the hardware exp2/rcp/log2 approximations, silu and softplus, and the
// grid of the grid-stride kernels. Included by exactly one translation unit
// per kernel family; everything has internal linkage.
#pragma once

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

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float fast_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// silu(z) = z / (1 + exp(-z))
__device__ __forceinline__ float silu(float z) {
    return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e));
}

constexpr float kLn2 = 0.69314718055994530942f;

// softplus(v) = log(1 + exp(v)) = max(v, 0) + log1p(e), e = exp(-|v|) in
// (0, 1]. log1p(e) is taken as log(w) * e / (w - 1) with w = 1 + e rounded
// (Goldberg, "What Every Computer Scientist Should Know About Floating-Point
// Arithmetic", Theorem 4): the rounding of w cancels between the two
// factors, so small e keep their relative accuracy instead of vanishing in
// log(w). Overflow cannot happen; NaN stays NaN.
__device__ __forceinline__ float softplus_f32(float v) {
    const float e = fast_exp2(-fabsf(v) * kLog2e);
    const float w = 1.0f + e;
    const float l = w == 1.0f ? e : __builtin_amdgcn_logf(w) * kLn2 * (e * fast_rcp(w - 1.0f));
    return fmaxf(v, 0.0f) + l;
}

// Half channel groups (the forward scan's and the backward pass's): the
// last channel groups of a launch can run as two halves of 32 channels, each
// channel's states spread over 8 lanes (two 32-lane rows per wave).
constexpr int kHalfChannels = 32;
constexpr int kHalfSplits = 8;

// Which split group and which half block `hb` of `nhb` half blocks runs.
// The two halves of a group read the two 64-byte halves of the same
// 128-byte rows, so they are placed 8 blocks apart, on one XCD (block i
// goes to XCD i mod 8) whose L2 then fetches those rows once: within every
// 16 half blocks, block r < 8 is half 0 and block 8 + r half 1 of the same
// group; a last partial run of blocks pairs neighbours.
__device__ __forceinline__ void half_block_pair(int64_t hb, int64_t nhb, int64_t& pair,
                                                int& side) {
    const int64_t run = hb / 16, r = hb % 16;
    if ((run + 1) * 16 <= nhb) {
        pair = run * 8 + r % 8;
        side = static_cast<int>(r / 8);
    } else {
        pair = hb / 2;
        side = static_cast<int>(hb % 2);
    }
}

// Workgroups are handed to the chip's 8 XCDs in turn (workgroup i to XCD
// i mod 8), and every XCD has its own L2. This maps the hardware workgroup
// id to a logical one such that each XCD runs one contiguous range of
// logical workgroups, so workgroups that are neighbours in the logical
// order, and read neighbouring data, share an L2. It is a bijection on
// [0, nblocks).
constexpr int64_t kXcds = 8;

__device__ __forceinline__ int64_t xcd_contiguous_block(int64_t bid, int64_t nblocks) {
    const int64_t q = nblocks / kXcds, r = nblocks % kXcds;
    const int64_t xcd = bid % kXcds, k = bid / kXcds;
    return xcd < r ? xcd * (q + 1) + k : r * (q + 1) + (xcd - r) * q + k;
}

// Grid for the grid-stride kernels above: enough 256-thread blocks to cover
// `count` items, capped well below the 32-bit grid limit.
inline int64_t stride_blocks(int64_t count) {
    const int64_t b = (count + 255) / 256;
    return b < (int64_t(1) << 20) ? (b > 0 ? b : 1) : (int64_t(1) << 20);
}

}  // namespace
}  // namespace mamba
