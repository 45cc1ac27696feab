// C ABI of the selective-scan library: argument checks, the chunk plan and
// error mapping around the HIP kernels (scan_variant.hip, launch.hip,
// scan_bwd.hip, ssd.hip, conv1d.hip).
//
// Every check runs on the host before any HIP call, so a rejected call
// queues nothing and leaves the device untouched. The only HIP calls outside
// the launches are the device and compute-unit-count queries of the
// automatic chunk plan; the compute-unit count of each device is queried
// once and kept for the life of the process (the only state the library
// holds besides the fixed scratch of ssm_scan_fwd_noalloc, noalloc.hip).
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <stdint.h>

#include "internal.h"
#include "mamba_scan.h"

namespace {

using mamba::ScanPlan;

static_assert(mamba::kConvMaxWidth == MAMBA_CONV_MAX_WIDTH, "convolution width limit");

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet

// Compute units of the current device (cached per device).
int current_cu_count(int* cu) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MAMBA_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) {
        const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
        if (cached > 0) {
            *cu = cached;
            return MAMBA_OK;
        }
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return MAMBA_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
    *cu = n;
    return MAMBA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Reads the optional delta transforms; NULL means none.
int read_options(const mamba_scan_options* o, const float** bias, int* softplus) {
    *bias = nullptr;
    *softplus = 0;
    if (o == nullptr) return MAMBA_OK;
    if (o->reserved != 0) return MAMBA_ERR_INVALID_ARG;
    if (o->delta_bias != nullptr && !aligned16(o->delta_bias)) return MAMBA_ERR_MISALIGNED;
    *bias = o->delta_bias;
    *softplus = o->delta_softplus != 0;
    return MAMBA_OK;
}

int check_shape(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int dtype) {
    if (batch < 0 || seqlen < 0 || dim < 0) return MAMBA_ERR_INVALID_ARG;
    if (dtype != MAMBA_DTYPE_F32 && dtype != MAMBA_DTYPE_BF16) return MAMBA_ERR_INVALID_ARG;
    if (dstate < 1 || dstate > MAMBA_SCAN_MAX_DSTATE) return MAMBA_ERR_UNSUPPORTED;
    // every element and workgroup index must fit comfortably in int64 / the grid
    const int64_t lim = int64_t(1) << 48;
    if (batch > lim || seqlen > lim || dim > lim) return MAMBA_ERR_UNSUPPORTED;
    // the (batch, dim, dstate) state and the decode grid stay far from overflow
    if (batch != 0 && dim > (int64_t(1) << 36) / batch) return MAMBA_ERR_UNSUPPORTED;
    if (batch != 0 && dim != 0 && seqlen != 0) {
        if (seqlen > lim / batch || batch * seqlen > lim / dim) return MAMBA_ERR_UNSUPPORTED;
    }
    return MAMBA_OK;
}

// Work decomposition. A workgroup of `state_split` waves scans 64 channels
// of one batch row over one chunk. The automatic plan splits every channel's
// states over four waves where the kernels allow it (dstate 4, 8 or 16):
// that multiplies the waves by four for about a sixth more vector work, far
// cheaper than cutting the sequence, where every chunk but the first and the
// last pays a summary pass. Only when the split launch still holds fewer
// than two waves per SIMD is the sequence cut. Chunks are never shorter than
// kMinChunk tokens. (Measured on MI355X for the Mamba-130M and Mamba-2.8B
// layer shapes.)
//
// How many chunks (rerun carry). Pass 1 (chunk 0's outputs and the
// summaries of chunks 1 .. n-2) and pass 2 (the outputs of chunks 1 .. n-1)
// each hold n-1 layers of the G channel groups. Both are bound by vector
// issue, so a pass takes about as long as its busiest compute unit: m =
// ceil((n-1) G / CU) workgroups of one chunk each, a summary costing about
// kSummaryCost of an output pass per token, and every workgroup some
// kChunkFixedTokens' worth of fixed cost (pipeline fill, prologue). Fewer
// than six resident workgroups per unit issue less often: measured on the
// Mamba-130M layer, three ran at 0.83 and four at 0.91 of the rate of six,
// taken as (m + 12) / 18. The plan takes the n that minimises
// (chunk_len + kChunkFixedTokens) * (m * kSummaryCost + (1 - kSummaryCost)
// + m) / rate(m) among those that leave both passes at least
// kWavesPerSimdChunked waves per SIMD, preferring fewer chunks unless more
// cost at least 1% less. (Mamba-130M layer, 192 groups on 256 units: 9
// chunks, six workgroups per unit in either pass, 142 us, against 150 us for
// 8 chunks, whose pass 1 left a quarter of the units a workgroup short, and
// 146 us for 5.)
//
// Chunks of kRepairMinChunk tokens or more join through the repaired carry:
// its rerun covers only a chunk's head while the entering state still
// counts, which on long chunks is a small part of the summary pass it
// replaces (the million-token scan: about 1,100 of 21,848 tokens). Short
// chunks keep the summary pass, since a rerun that covers the whole chunk
// costs more than the summary. Without a summary pass more chunks cost only
// their head reruns, so such plans aim at about eight waves per SIMD (the
// million-token scan: 7.99 ms with 64 chunks against 8.16 ms with 48).
constexpr int kPreferredSplit = 4;
constexpr int64_t kRepairMinChunk = 4096;
static_assert(mamba::kCarryRerun == MAMBA_CARRY_RERUN && mamba::kCarryRepair == MAMBA_CARRY_REPAIR,
              "internal carry codes follow the public enum");
constexpr int64_t kWavesPerSimdNoChunk = 2;
constexpr int64_t kWavesPerSimdChunked = 3;
constexpr int64_t kWavesPerSimdRepaired = 8;
constexpr int64_t kMinChunk = 64;
constexpr double kSummaryCost = 0.75;
constexpr double kChunkFixedTokens = 32.0;

// Chunk length of `n` chunks over seqlen tokens, a whole number of tiles.
int64_t chunk_len_for(int64_t seqlen, int64_t n) {
    const int64_t c = (seqlen + n - 1) / n;
    return (c + mamba::kTokenTile - 1) / mamba::kTokenTile * mamba::kTokenTile;
}

// The rerun carry's chunk length by the balance rule above. When no count
// leaves enough waves per SIMD (very few channel groups), the most chunks
// the minimum length allows: the passes are then bound by latency, which
// shorter chunks cut.
int64_t rerun_chunk_len(int64_t seqlen, int64_t groups, int split, int cu) {
    const int64_t nmax = seqlen / kMinChunk;
    int64_t best_len = chunk_len_for(seqlen, nmax);
    double best = -1.0;
    // counts below n0 leave too few waves per SIMD; the cost repeats its
    // pattern every CU / gcd(G, CU) counts, so a window of 4 CU counts past
    // n0 holds the minimum
    const int64_t need = kWavesPerSimdChunked * 4 * int64_t(cu);
    const int64_t n0 = 1 + (need + groups * split - 1) / (groups * split);
    const int64_t n1 = nmax < n0 + 4 * int64_t(cu) ? nmax : n0 + 4 * int64_t(cu);
    for (int64_t n = n0 > 2 ? n0 : 2; n <= n1; ++n) {
        const int64_t len = chunk_len_for(seqlen, n);
        const int64_t chunks = (seqlen + len - 1) / len;
        if (chunks != n) continue;  // rounding to whole tiles merged two counts
        const int64_t layers = (n - 1) * groups;
        if (layers * split < kWavesPerSimdNoChunk * 4 * int64_t(cu)) continue;
        const double m = static_cast<double>((layers + cu - 1) / cu);
        const double rate = m >= 6.0 ? 1.0 : (m + 12.0) / 18.0;
        const double cost = (static_cast<double>(len) + kChunkFixedTokens) *
                            (m * kSummaryCost + (1.0 - kSummaryCost) + m) / rate;
        if (best < 0.0 || cost < 0.99 * best) {
            best = cost;
            best_len = len;
        }
    }
    return best_len;
}

int make_plan(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int dtype,
              const mamba_scan_plan* req, ScanPlan* plan) {
    int64_t len = req ? req->chunk_len : 0;
    int split = req ? req->state_split : 0;
    const int carry = req ? req->carry : MAMBA_CARRY_AUTO;
    const int64_t halves = req ? req->halves : 0;
    if (carry != MAMBA_CARRY_AUTO && carry != MAMBA_CARRY_RERUN && carry != MAMBA_CARRY_REPAIR)
        return MAMBA_ERR_INVALID_ARG;
    if ((req && req->reserved != 0) || halves < -1) return MAMBA_ERR_INVALID_ARG;
    if (len < 0 || split < 0) return MAMBA_ERR_INVALID_ARG;
    if (split != 0 && !mamba::split_supported(dstate, split)) return MAMBA_ERR_UNSUPPORTED;
    if (seqlen == 0 || batch == 0 || dim == 0) {
        plan->chunk_len = seqlen;
        plan->nchunks = 1;
        plan->state_split = split ? split : 1;
        plan->carry = carry != MAMBA_CARRY_AUTO ? carry : MAMBA_CARRY_RERUN;
        plan->halves = 0;  // nothing runs: any request is moot
        plan->workspace_bytes = 0;
        return MAMBA_OK;
    }
    const int64_t groups = batch * ((dim + mamba::kWave - 1) / mamba::kWave);
    if (split == 0 || len == 0) {
        int cu = 0;
        const int st = current_cu_count(&cu);
        if (st != MAMBA_OK) return st;
        const int64_t simds = int64_t(cu) * 4;
        if (split == 0) {
            split = 1;
            for (int sp = kPreferredSplit; sp > 1; sp /= 2)
                if (mamba::split_supported(dstate, sp)) {
                    split = sp;
                    break;
                }
        }
        if (len == 0) {
            const int64_t waves = groups * split;
            const int64_t nmax = seqlen / kMinChunk;
            len = seqlen;
            if (waves < kWavesPerSimdNoChunk * simds && nmax >= 2) {
                len = rerun_chunk_len(seqlen, groups, split, cu);
                // chunks that will join through the repaired carry: about
                // eight waves per SIMD, when that keeps them long
                if (carry != MAMBA_CARRY_RERUN) {
                    int64_t n = (kWavesPerSimdRepaired * simds + waves - 1) / waves;
                    if (n > nmax) n = nmax;
                    const int64_t longer = chunk_len_for(seqlen, n < 1 ? 1 : n);
                    if (longer >= kRepairMinChunk && longer < seqlen) len = longer;
                }
            }
        }
    }
    if (len > seqlen) len = seqlen;
    // a chunk's x/delta/z/y rows (dim per token) and B/C rows (dstate per
    // token) are addressed with 32-bit byte offsets: its extent over the
    // wider of the two stays below 2^32 bytes
    const int64_t esz = dtype == MAMBA_DTYPE_F32 ? 4 : 2;
    const int64_t row = dim > dstate ? dim : dstate;
    const int64_t max_len = ((int64_t(1) << 32) - 1) / (row * esz);
    if (max_len < 1) return MAMBA_ERR_UNSUPPORTED;
    if (len > max_len) len = max_len;
    const int64_t nchunks = (seqlen + len - 1) / len;
    if (groups > (int64_t(1) << 31) / nchunks) return MAMBA_ERR_UNSUPPORTED;
    plan->chunk_len = len;
    plan->nchunks = nchunks;
    plan->state_split = split;
    plan->carry = carry != MAMBA_CARRY_AUTO
                      ? carry
                      : (nchunks > 1 && len >= kRepairMinChunk ? MAMBA_CARRY_REPAIR
                                                               : MAMBA_CARRY_RERUN);
    plan->workspace_bytes = mamba::scan_workspace_bytes(batch, dim, dstate, nchunks);
    // whole and half channel groups
    plan->halves = 0;
    const bool halvable = nchunks == 1 && split == 4 && (dstate == 8 || dstate == 16);
    if (halves > 0) {
        if (!halvable) return MAMBA_ERR_UNSUPPORTED;
        if (halves > groups) return MAMBA_ERR_INVALID_ARG;
        plan->halves = halves;
    } else if (halves == 0 && halvable) {
        int cu = 0;
        const int st = current_cu_count(&cu);
        if (st != MAMBA_OK) return st;
        const int64_t surplus = groups % cu;
        if (surplus > 0 && 2 * surplus <= cu) plan->halves = surplus;
    }
    // the launch holds the whole groups and two blocks per split group
    if (groups + plan->halves > (int64_t(1) << 31)) return MAMBA_ERR_UNSUPPORTED;
    return MAMBA_OK;
}

}  // namespace

extern "C" {

int ssm_scan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int dstate,
                                int dtype, const mamba_scan_plan* request,
                                mamba_scan_plan* resolved, size_t* bytes) {
    if (bytes == nullptr) return MAMBA_ERR_INVALID_ARG;
    const int st = check_shape(batch, seqlen, dim, dstate, dtype);
    if (st != MAMBA_OK) return st;
    ScanPlan plan;
    const int ps = make_plan(batch, seqlen, dim, dstate, dtype, request, &plan);
    if (ps != MAMBA_OK) return ps;
    *bytes = plan.workspace_bytes;
    if (resolved != nullptr) {
        resolved->chunk_len = plan.chunk_len;
        resolved->state_split = plan.state_split;
        resolved->carry = plan.carry;
        resolved->halves = static_cast<int32_t>(plan.halves);
        resolved->reserved = 0;
    }
    return MAMBA_OK;
}

}  // extern "C"

namespace mamba {

// ssm_scan_fwd's checks, plan and launch. With `scratch` the workspace is
// not an argument: once the plan is known and needs one, scratch() is asked
// for it (after every argument check, so a rejected call makes no HIP call).
int scan_fwd_call(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int dtype,
                  const void* x, const void* delta, const float* A, const void* B,
                  const void* C, const float* D, const void* z, const float* h0, void* y,
                  float* hL, const mamba_scan_options* options,
                  const mamba_scan_plan* plan_req, void* workspace, size_t workspace_bytes,
                  ScratchSource scratch, hipStream_t stream) {
    int st = check_shape(batch, seqlen, dim, dstate, dtype);
    if (st != MAMBA_OK) return st;
    const float* delta_bias = nullptr;
    int delta_softplus = 0;
    st = read_options(options, &delta_bias, &delta_softplus);
    if (st != MAMBA_OK) return st;
    if (batch == 0 || dim == 0) return MAMBA_OK;
    if (A == nullptr) return MAMBA_ERR_INVALID_ARG;
    if (seqlen > 0 && (x == nullptr || delta == nullptr || B == nullptr || C == nullptr ||
                       y == nullptr))
        return MAMBA_ERR_INVALID_ARG;
    const void* ptrs[] = {x, delta, A, B, C, D, z, h0, y, hL, workspace};
    for (const void* p : ptrs)
        if (p != nullptr && !aligned16(p)) return MAMBA_ERR_MISALIGNED;
    if (seqlen == 0 && hL == nullptr) return MAMBA_OK;

    ScanPlan plan;
    st = make_plan(batch, seqlen, dim, dstate, dtype, plan_req, &plan);
    if (st != MAMBA_OK) return st;
    if (scratch != nullptr && plan.workspace_bytes > 0) {
        st = scratch(plan.workspace_bytes, &workspace);
        if (st != MAMBA_OK) return st;
        workspace_bytes = plan.workspace_bytes;
    }
    if (plan.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.workspace_bytes))
        return MAMBA_ERR_WORKSPACE;

    ScanArgs a;
    a.batch = batch;
    a.seqlen = seqlen;
    a.dim = dim;
    a.dstate = dstate;
    a.io = dtype == MAMBA_DTYPE_F32 ? kIoF32 : kIoBF16;
    a.x = x;
    a.delta = delta;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.z = z;
    a.h0 = h0;
    a.y = y;
    a.hL = hL;
    a.delta_bias = delta_bias;
    a.delta_softplus = delta_softplus;
    return launch_scan(a, plan, workspace, stream) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

}  // namespace mamba

extern "C" {

int ssm_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int dtype,
                 const void* x, const void* delta, const float* A, const void* B,
                 const void* C, const float* D, const void* z, const float* h0, void* y,
                 float* hL, const mamba_scan_options* options,
                 const mamba_scan_plan* plan_req, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
    return mamba::scan_fwd_call(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, D, z, h0,
                                y, hL, options, plan_req, workspace, workspace_bytes, nullptr,
                                stream);
}

int ssm_state_update(int64_t batch, int64_t dim, int dstate, int dtype, float* h,
                     const void* x, const void* delta, const float* A, const void* B,
                     const void* C, const float* D, const void* z, void* y,
                     const mamba_scan_options* options, hipStream_t stream) {
    int st = check_shape(batch, 1, dim, dstate, dtype);
    if (st != MAMBA_OK) return st;
    const float* delta_bias = nullptr;
    int delta_softplus = 0;
    st = read_options(options, &delta_bias, &delta_softplus);
    if (st != MAMBA_OK) return st;
    if (batch == 0 || dim == 0) return MAMBA_OK;
    if (h == nullptr || x == nullptr || delta == nullptr || A == nullptr || B == nullptr ||
        C == nullptr || y == nullptr)
        return MAMBA_ERR_INVALID_ARG;
    const void* ptrs[] = {h, x, delta, A, B, C, D, z, y};
    for (const void* p : ptrs)
        if (p != nullptr && !aligned16(p)) return MAMBA_ERR_MISALIGNED;

    mamba::DecodeArgs a;
    a.batch = batch;
    a.dim = dim;
    a.dstate = dstate;
    a.io = dtype == MAMBA_DTYPE_F32 ? mamba::kIoF32 : mamba::kIoBF16;
    a.h = h;
    a.x = x;
    a.delta = delta;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.z = z;
    a.y = y;
    a.delta_bias = delta_bias;
    a.delta_softplus = delta_softplus;
    return mamba::launch_state_update(a, stream) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

}  // extern "C"

namespace {

// Work decomposition of the backward pass. One workgroup of ceil(N/4) waves
// walks one (chunk, batch row, 64-channel group). The sequence stays whole
// unless the groups' waves fill less than kWavesPerSimdNoChunk waves per
// SIMD; it is then cut into chunks of at least kMinChunk tokens for about
// kBwdWavesPerSimd waves per SIMD (two rounds of the three the kernel holds
// per SIMD), at the price of a state and an adjoint summary over every chunk
// but one. (Measured on MI355X: the Mamba-130M layer 0.50 ms with 8 chunks,
// 0.51-0.53 ms with 6, 7, 9, 10, 12 or 16; the Mamba-2.8B layer, whose 640
// groups fill 2.5 waves per SIMD, 1.35 ms whole against 1.47-1.55 ms with
// 2 to 8 chunks.) Halves
// (the last groups as two 32-channel halves, as in the forward plan) need
// a whole sequence: forced halves keep it whole.
constexpr int64_t kBwdWavesPerSimd = 6;

// The checks of a requested backward plan that need no device.
int check_bwd_plan(int64_t batch, int64_t seqlen, int64_t dim, int dstate,
                   const mamba_scan_plan* req) {
    if (req == nullptr) return MAMBA_OK;
    if (req->state_split != 0 || req->carry != 0 || req->reserved != 0 || req->halves < -1 ||
        req->chunk_len < 0 || req->chunk_len % 8 != 0)
        return MAMBA_ERR_INVALID_ARG;
    if (batch <= 0 || seqlen <= 0 || dim <= 0) return MAMBA_OK;  // nothing runs: moot
    const int64_t groups = batch * ((dim + mamba::kWave - 1) / mamba::kWave);
    if (req->halves > 0 && !mamba::bwd_halves_supported(dstate)) return MAMBA_ERR_UNSUPPORTED;
    if (req->halves > groups) return MAMBA_ERR_INVALID_ARG;
    const bool chunked = req->chunk_len > 0 && req->chunk_len < seqlen;
    if (chunked && req->halves > 0) return MAMBA_ERR_UNSUPPORTED;
    return MAMBA_OK;
}

// The backward plan: chunk length (0: one chunk) and halves. Automatic
// fields query the current device.
int make_bwd_plan(int64_t batch, int64_t seqlen, int64_t dim, int dstate,
                  const mamba_scan_plan* req, int64_t* chunk_len, int64_t* halves) {
    const int st = check_bwd_plan(batch, seqlen, dim, dstate, req);
    if (st != MAMBA_OK) return st;
    const int64_t len_req = req != nullptr ? req->chunk_len : 0;
    const int64_t halves_req = req != nullptr ? req->halves : 0;
    *chunk_len = 0;
    *halves = 0;
    if (batch <= 0 || seqlen <= 0 || dim <= 0) return MAMBA_OK;
    const int64_t groups = batch * ((dim + mamba::kWave - 1) / mamba::kWave);
    int cu = 0;
    if (len_req == 0 || halves_req == 0) {
        const int st = current_cu_count(&cu);
        if (st != MAMBA_OK) return st;
    }
    int64_t len = len_req;
    if (len == 0 && halves_req <= 0) {  // forced halves keep the sequence whole
        const int64_t waves = groups * ((dstate + 3) / 4);
        const int64_t simds = int64_t(cu) * 4;
        if (waves < kWavesPerSimdNoChunk * simds) {
            int64_t n = (kBwdWavesPerSimd * simds + waves - 1) / waves;
            if (n > seqlen / kMinChunk) n = seqlen / kMinChunk;
            if (n >= 2) len = ((seqlen + n - 1) / n + 7) / 8 * 8;
        }
    }
    if (len >= seqlen) len = 0;  // one chunk
    const int64_t nchunks = len > 0 ? (seqlen + len - 1) / len : 1;
    if (nchunks > 1 && halves_req > 0) return MAMBA_ERR_UNSUPPORTED;
    if (nchunks == 1 && mamba::bwd_halves_supported(dstate)) {
        if (halves_req > 0) {
            *halves = halves_req;
        } else if (halves_req == 0) {
            // the groups whole rounds leave over, when at most half a round
            const int64_t surplus = groups % cu;
            if (surplus > 0 && 2 * surplus <= cu) *halves = surplus;
        }
    }
    // the largest launch: both chunk summaries together, or the main kernel
    if (2 * nchunks * groups + *halves > (int64_t(1) << 31)) return MAMBA_ERR_UNSUPPORTED;
    *chunk_len = len;
    return MAMBA_OK;
}

}  // namespace

extern "C" {

int ssm_scan_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int dstate,
                                int dtype, const mamba_scan_plan* plan,
                                mamba_scan_plan* resolved, size_t* bytes) {
    if (bytes == nullptr) return MAMBA_ERR_INVALID_ARG;
    int st = check_shape(batch, seqlen, dim, dstate, dtype);
    if (st != MAMBA_OK) return st;
    int64_t chunk_len = 0, halves = 0;
    st = make_bwd_plan(batch, seqlen, dim, dstate, plan, &chunk_len, &halves);
    if (st != MAMBA_OK) return st;
    *bytes = mamba::scan_bwd_workspace_bytes(batch, seqlen, dim, dstate, chunk_len);
    if (resolved != nullptr) {
        *resolved = mamba_scan_plan{};
        resolved->chunk_len = chunk_len > 0 ? chunk_len : seqlen;
        resolved->halves = halves;
    }
    return MAMBA_OK;
}

int ssm_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int dtype,
                 const void* x, const void* delta, const float* A, const void* B,
                 const void* C, const float* D, const void* z, const float* h0,
                 const mamba_scan_options* options, const mamba_scan_plan* plan,
                 const void* dy, const float* dhL,
                 void* dx, void* ddelta, float* dA, float* dB, float* dC, float* dD,
                 void* dz, float* dh0, float* ddelta_bias, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
    int st = check_shape(batch, seqlen, dim, dstate, dtype);
    if (st != MAMBA_OK) return st;
    st = check_bwd_plan(batch, seqlen, dim, dstate, plan);
    if (st != MAMBA_OK) return st;
    const float* delta_bias = nullptr;
    int delta_softplus = 0;
    st = read_options(options, &delta_bias, &delta_softplus);
    if (st != MAMBA_OK) return st;
    if ((dD != nullptr && D == nullptr) || (dz != nullptr && z == nullptr) ||
        (ddelta_bias != nullptr && delta_bias == nullptr))
        return MAMBA_ERR_INVALID_ARG;
    if (dim == 0) return MAMBA_OK;
    if (A == nullptr || dA == nullptr) return MAMBA_ERR_INVALID_ARG;
    if (batch > 0 && seqlen > 0 &&
        (x == nullptr || delta == nullptr || B == nullptr || C == nullptr || dy == nullptr ||
         dx == nullptr || ddelta == nullptr || dB == nullptr || dC == nullptr))
        return MAMBA_ERR_INVALID_ARG;
    const void* ptrs[] = {x, delta, A, B, C, D, z, h0, dy, dhL, dx, ddelta,
                          dA, dB, dC, dD, dz, dh0, ddelta_bias, workspace};
    for (const void* p : ptrs)
        if (p != nullptr && !aligned16(p)) return MAMBA_ERR_MISALIGNED;
    int64_t chunk_len = 0, halves = 0;
    st = make_bwd_plan(batch, seqlen, dim, dstate, plan, &chunk_len, &halves);
    if (st != MAMBA_OK) return st;
    const size_t need = mamba::scan_bwd_workspace_bytes(batch, seqlen, dim, dstate, chunk_len);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return MAMBA_ERR_WORKSPACE;
    mamba::BwdArgs a;
    a.halves = halves;
    a.chunk_len = chunk_len;
    a.fwd.batch = batch;
    a.fwd.seqlen = seqlen;
    a.fwd.dim = dim;
    a.fwd.dstate = dstate;
    a.fwd.io = dtype == MAMBA_DTYPE_F32 ? mamba::kIoF32 : mamba::kIoBF16;
    a.fwd.x = x;
    a.fwd.delta = delta;
    a.fwd.A = A;
    a.fwd.B = B;
    a.fwd.C = C;
    a.fwd.D = D;
    a.fwd.z = z;
    a.fwd.h0 = h0;
    a.fwd.y = nullptr;
    a.fwd.hL = nullptr;
    a.fwd.delta_bias = delta_bias;
    a.fwd.delta_softplus = delta_softplus;
    a.dy = dy;
    a.dhL = dhL;
    a.dx = dx;
    a.ddelta = ddelta;
    a.dA = dA;
    a.dB = dB;
    a.dC = dC;
    a.dD = dD;
    a.dz = dz;
    a.dh0 = dh0;
    a.ddelta_bias = ddelta_bias;
    return mamba::launch_scan_bwd(a, workspace, stream) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

int ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int dstate,
            int dtype, const void* x, const void* dt, const float* A, const void* B,
            const void* C, const float* D, const void* z, const float* h0, void* y, float* hL,
            const mamba_scan_options* options, hipStream_t stream) {
    if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 0) return MAMBA_ERR_INVALID_ARG;
    if (dtype != MAMBA_DTYPE_F32 && dtype != MAMBA_DTYPE_BF16) return MAMBA_ERR_INVALID_ARG;
    if (headdim != MAMBA_SSD_HEADDIM || (dstate != 64 && dstate != 128) ||
        dtype != MAMBA_DTYPE_BF16)
        return MAMBA_ERR_UNSUPPORTED;
    if (nheads > (int64_t(1) << 16)) return MAMBA_ERR_UNSUPPORTED;
    int st = check_shape(batch, seqlen, nheads * headdim, 1, dtype);
    if (st != MAMBA_OK) return st;
    if (batch * nheads >= (int64_t(1) << 31)) return MAMBA_ERR_UNSUPPORTED;
    const float* dt_bias = nullptr;
    int dt_softplus = 0;
    st = read_options(options, &dt_bias, &dt_softplus);
    if (st != MAMBA_OK) return st;
    if (batch == 0 || nheads == 0) return MAMBA_OK;
    if (A == nullptr) return MAMBA_ERR_INVALID_ARG;
    if (seqlen > 0 && (x == nullptr || dt == nullptr || B == nullptr || C == nullptr ||
                       y == nullptr))
        return MAMBA_ERR_INVALID_ARG;
    const void* ptrs[] = {x, dt, A, B, C, D, z, h0, y, hL};
    for (const void* p : ptrs)
        if (p != nullptr && !aligned16(p)) return MAMBA_ERR_MISALIGNED;
    if (seqlen == 0 && hL == nullptr) return MAMBA_OK;

    mamba::SsdArgs a;
    a.batch = batch;
    a.seqlen = seqlen;
    a.nheads = nheads;
    a.dstate = dstate;
    a.x = x;
    a.dt = dt;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.z = z;
    a.h0 = h0;
    a.y = y;
    a.hL = hL;
    a.dt_bias = dt_bias;
    a.dt_softplus = dt_softplus;
    return mamba::launch_ssd_fwd(a, stream) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

int causal_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int width, int dtype,
                      const void* x, const float* weight, const float* bias,
                      const void* state_in, void* y, void* state_out, int silu,
                      hipStream_t stream) {
    int st = check_shape(batch, seqlen, dim, 1, dtype);
    if (st != MAMBA_OK) return st;
    if (width < 1 || width > MAMBA_CONV_MAX_WIDTH) return MAMBA_ERR_UNSUPPORTED;
    if (batch == 0 || dim == 0) return MAMBA_OK;
    if (weight == nullptr) return MAMBA_ERR_INVALID_ARG;
    if (seqlen > 0 && (x == nullptr || y == nullptr)) return MAMBA_ERR_INVALID_ARG;
    const void* ptrs[] = {x, weight, bias, state_in, y, state_out};
    for (const void* p : ptrs)
        if (p != nullptr && !aligned16(p)) return MAMBA_ERR_MISALIGNED;
    if (seqlen == 0 && state_out == nullptr) return MAMBA_OK;

    mamba::ConvArgs a;
    a.batch = batch;
    a.seqlen = seqlen;
    a.dim = dim;
    a.width = width;
    a.io = dtype == MAMBA_DTYPE_F32 ? mamba::kIoF32 : mamba::kIoBF16;
    a.silu = silu != 0;
    a.x = x;
    a.weight = weight;
    a.bias = bias;
    a.state_in = state_in;
    a.y = y;
    a.state_out = state_out;
    a.fuse_state = 0;
    return mamba::launch_conv1d(a, false, stream) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

int causal_conv1d_update(int64_t batch, int64_t dim, int width, int dtype, void* state,
                         const void* x, const float* weight, const float* bias, void* y,
                         int silu, hipStream_t stream) {
    int st = check_shape(batch, 1, dim, 1, dtype);
    if (st != MAMBA_OK) return st;
    if (width < 1 || width > MAMBA_CONV_MAX_WIDTH) return MAMBA_ERR_UNSUPPORTED;
    if (batch == 0 || dim == 0) return MAMBA_OK;
    if (state == nullptr || x == nullptr || weight == nullptr || y == nullptr)
        return MAMBA_ERR_INVALID_ARG;
    const void* ptrs[] = {state, x, weight, bias, y};
    for (const void* p : ptrs)
        if (p != nullptr && !aligned16(p)) return MAMBA_ERR_MISALIGNED;

    mamba::ConvArgs a;
    a.batch = batch;
    a.seqlen = 1;
    a.dim = dim;
    a.width = width;
    a.io = dtype == MAMBA_DTYPE_F32 ? mamba::kIoF32 : mamba::kIoBF16;
    a.silu = silu != 0;
    a.x = x;
    a.weight = weight;
    a.bias = bias;
    a.state_in = state;
    a.y = y;
    a.state_out = state;
    a.fuse_state = 0;
    return mamba::launch_conv1d(a, true, stream) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

const char* mamba_status_string(int status) {
    switch (status) {
        case MAMBA_OK: return "MAMBA_OK: success";
        case MAMBA_ERR_INVALID_ARG: return "MAMBA_ERR_INVALID_ARG: invalid argument";
        case MAMBA_ERR_UNSUPPORTED:
            return "MAMBA_ERR_UNSUPPORTED: unsupported size, dstate, split or width";
        case MAMBA_ERR_MISALIGNED: return "MAMBA_ERR_MISALIGNED: pointer not 16-byte aligned";
        case MAMBA_ERR_WORKSPACE: return "MAMBA_ERR_WORKSPACE: workspace missing or too small";
        case MAMBA_ERR_HIP: return "MAMBA_ERR_HIP: HIP runtime error";
        default: return "unknown mamba_status";
    }
}

}  // extern "C"
