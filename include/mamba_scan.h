/*
 * mamba_scan.h: C ABI of the selective state-space scan for AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (page "Mamba and State Space Models", world.lapla.si):
 * for every batch row b, channel d and state n, with A[d,n] < 0,
 *
 *     Abar = exp(delta[b,t,d] * A[d,n])                 ("Chosen by the Token")
 *     h[n] <- Abar * h[n] + delta[b,t,d] * B[b,t,n] * x[b,t,d]
 *                                                       ("A State of Fixed Size")
 *     y[b,t,d] = (sum_n C[b,t,n] * h[n] + D[d] * x[b,t,d]) * silu(z[b,t,d])
 *
 * with silu(z) = z / (1 + exp(-z)). The output of token t reads the state
 * after token t has been absorbed. The input discretisation is the
 * first-order form Bbar = delta * B; the skip term D*x and the silu gate are
 * optional. Delta, B and C arrive computed per token (section "Chosen by the
 * Token"). Delta must be positive (not checked); it may also arrive before
 * its activation, see mamba_scan_options.
 *
 * Layout: every tensor is dense and row-major.
 *     x, delta, z, y   (batch, seqlen, dim)      dim contiguous, I/O dtype
 *     B, C             (batch, seqlen, dstate)   I/O dtype, shared by all channels
 *     A                (dim, dstate)             fp32
 *     D                (dim)                     fp32
 *     h0, hL, h        (batch, dim, dstate)      fp32
 * The I/O dtype (MAMBA_DTYPE_F32 or MAMBA_DTYPE_BF16) applies to x, delta,
 * z, B, C and y. The state is always fp32 and all arithmetic is fp32.
 *
 * Ownership and threading: all pointers are device pointers on the current
 * HIP device, owned by the caller. The library keeps no pointer after a call
 * returns and allocates no device memory; ssm_scan_fwd takes its scratch
 * space from the caller's workspace. Work is queued on `stream` (0 = the
 * null stream) and the call returns before it finishes, so buffers must
 * outlive the queued work. Calls on different streams do not share state,
 * with two exceptions: the automatic plans query each device's compute-unit
 * count once and keep it for the life of the process (a per-device cache
 * that threads may fill concurrently; it never changes), and
 * ssm_scan_fwd_noalloc's fixed scratch (see there).
 *
 * Errors: shape, dtype, null-pointer, alignment and workspace checks run on
 * the host before any HIP call and return a negative mamba_status; nothing
 * is queued then. A failed launch returns MAMBA_ERR_HIP. The library never
 * prints or aborts. Every pointer must be 16-byte aligned.
 */
#ifndef MAMBA_SCAN_H
#define MAMBA_SCAN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest supported number of states per channel (the pages' default is 16). */
#define MAMBA_SCAN_MAX_DSTATE 16

typedef enum mamba_status {
    MAMBA_OK = 0,
    MAMBA_ERR_INVALID_ARG = -1,   /* negative size, NULL required pointer, bad dtype */
    MAMBA_ERR_UNSUPPORTED = -2,   /* dstate outside 1..MAMBA_SCAN_MAX_DSTATE, sizes too large,
                                     a state split the kernels do not provide, a
                                     convolution width outside 1..MAMBA_CONV_MAX_WIDTH */
    MAMBA_ERR_MISALIGNED = -3,    /* a pointer is not 16-byte aligned */
    MAMBA_ERR_WORKSPACE = -4,     /* workspace NULL or smaller than required */
    MAMBA_ERR_HIP = -5            /* the HIP runtime reported an error */
} mamba_status;

typedef enum mamba_dtype {
    MAMBA_DTYPE_F32 = 0,
    MAMBA_DTYPE_BF16 = 1
} mamba_dtype;

/*
 * How chunks of a cut sequence learn the state entering them.
 *
 * MAMBA_CARRY_RERUN   a first pass runs chunk 0 to its outputs (from h0, so
 *                     its end state is exact) and summarises chunks 1 ..
 *                     n-2 from a zero state as (decay product, end state)
 *                     pairs; an associative combine of the pairs gives the
 *                     state entering each later chunk (the "parallel scan"
 *                     of section "A Scan on the Chip"), and a second pass
 *                     reruns chunks 1 .. n-1 from their entering states.
 * MAMBA_CARRY_REPAIR  every chunk runs once from a zero state (the first
 *                     from h0), writing y and its pair; the combine gives the
 *                     entering states and hL; each later chunk then reruns
 *                     from its entering state only until exp(A * sum of
 *                     delta since the chunk start) is at most 2^-32 for every
 *                     state of its 64-channel group, and keeps the zero-start
 *                     y after that. The outputs it keeps differ from the
 *                     rerun ones by less than 2^-32 * sum_n |C[n] h_in[n]|
 *                     (h_in: the entering state), below fp32 rounding of
 *                     that readout. The rerun length depends on the data: a
 *                     chunk whose decay never gets there (A >= 0, delta = 0,
 *                     a non-finite entering state) is rerun whole. The bound
 *                     rests on the weight only shrinking, i.e. on the
 *                     positive delta the scan requires (after the bias and
 *                     activation, when fused); with negative deltas only
 *                     MAMBA_CARRY_RERUN keeps the plain recurrence.
 */
typedef enum mamba_carry {
    MAMBA_CARRY_AUTO = 0,
    MAMBA_CARRY_RERUN = 1,
    MAMBA_CARRY_REPAIR = 2
} mamba_carry;

/*
 * How ssm_scan_fwd divides its work over the GPU (ssm_scan_bwd takes the
 * same struct and uses chunk_len and halves, as documented there). A NULL
 * plan, or a zero field, lets the library choose from the shape and the
 * current device's compute-unit count; every choice gives the same result
 * up to rounding (and, with MAMBA_CARRY_REPAIR, the bound stated above).
 *
 * chunk_len    tokens per parallel chunk. Each sequence is cut into chunks
 *              that run in parallel and are joined as `carry` says; when
 *              chunk_len does not divide seqlen, the first chunk is the
 *              shorter one. A chunk_len of seqlen or more means one chunk
 *              and a single pass. The library may shorten a chunk so a
 *              chunk of one channel group spans less than 4 GiB.
 * state_split  waves sharing the dstate states of each channel: 1, 2, 4 or
 *              8. Values above 1 need dstate of 4, 8 or 16 divisible by the
 *              split.
 * carry        a mamba_carry value; automatic picks MAMBA_CARRY_REPAIR for
 *              chunks of 4096 tokens or more, MAMBA_CARRY_RERUN otherwise.
 *              Ignored with one chunk. Other values: MAMBA_ERR_INVALID_ARG.
 * halves       channel groups (64 channels of one batch row) run as two
 *              halves of 32 channels, each channel's states then spread over
 *              8 lanes: the last `halves` groups in (row, group) order. It
 *              evens out the work per compute unit when the groups do not
 *              divide over the units (G groups on C units, G mod C <= C/2:
 *              every unit then holds G div C groups and at most one half).
 *              0: automatic (exactly that case); -1: none; k > 0: the last
 *              k groups (k at most the number of groups, else
 *              MAMBA_ERR_INVALID_ARG). Halves need one chunk, state_split 4
 *              and dstate 8 or 16; k > 0 on any other plan returns
 *              MAMBA_ERR_UNSUPPORTED, and automatic means none there.
 *              A resolved plan reports the number of groups split.
 * reserved     must be 0.
 */
typedef struct mamba_scan_plan {
    int64_t chunk_len;
    int32_t state_split;
    int32_t carry;
    int32_t halves;
    int32_t reserved;
} mamba_scan_plan;

/*
 * Optional transforms applied inside the kernels (a NULL options pointer
 * turns all of them off).
 *
 * delta_bias      (dim) fp32 device pointer or NULL: added to delta before
 *                 anything else uses it.
 * delta_softplus  nonzero: delta <- softplus(delta + bias), with
 *                 softplus(v) = log(1 + exp(v)). The pages have delta come
 *                 from a projection of the token and require it positive
 *                 (section "Chosen by the Token"); softplus is the activation
 *                 that makes it so, and fusing it saves a full pass over
 *                 delta. The activated delta feeds both exp(delta*A) and
 *                 delta*B*x.
 * reserved        must be 0.
 */
typedef struct mamba_scan_options {
    const float* delta_bias;
    int32_t delta_softplus;
    int32_t reserved;
} mamba_scan_options;

/*
 * Resolve the plan ssm_scan_fwd will use for this shape and report the
 * scratch bytes it needs (0 when the plan has a single chunk).
 *
 * request   the caller's plan (may be NULL: automatic)
 * resolved  receives the plan with every field decided (may be NULL)
 * bytes     receives the workspace size (required)
 * May query the current device (a HIP call) when a field is automatic.
 */
int ssm_scan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int dstate,
                                int dtype, const mamba_scan_plan* request,
                                mamba_scan_plan* resolved, size_t* bytes);

/*
 * Selective scan over whole sequences (prefill).
 *
 * x, delta   (batch, seqlen, dim)     required
 * A          (dim, dstate) fp32       required, A < 0 (not checked)
 * B, C       (batch, seqlen, dstate)  required
 * D          (dim) fp32               optional (NULL: no skip term)
 * z          (batch, seqlen, dim)     optional (NULL: no gate)
 * h0         (batch, dim, dstate)     optional (NULL: zero initial state)
 * y          (batch, seqlen, dim)     written
 * hL         (batch, dim, dstate)     optional, written with the state after
 *                                     the last token; may alias h0
 * options    delta bias and activation (may be NULL: none), see
 *            mamba_scan_options
 * plan       work division (may be NULL: automatic), see mamba_scan_plan
 * workspace  at least the bytes ssm_scan_fwd_workspace_size reports for the
 *            same shape and plan; may be NULL when that size is 0; its
 *            contents need no initialisation
 * seqlen == 0 writes hL = h0 (or zeros) and no y; batch == 0 or dim == 0 is
 * a no-op. y must not overlap any input.
 */
int ssm_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int dtype,
                 const void* x, const void* delta, const float* A,
                 const void* B, const void* C, const float* D, const void* z,
                 const float* h0, void* y, float* hL,
                 const mamba_scan_options* options, const mamba_scan_plan* plan,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Scratch bytes each GPU holds for ssm_scan_fwd_noalloc (32 MiB). */
#define MAMBA_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * ssm_scan_fwd without a workspace argument. It allocates nothing (no
 * hipMalloc, hipFree or allocating library call). A plan that needs scratch
 * (a chunked sequence) takes it from a fixed array of
 * MAMBA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends; the first such call on a device looks up that
 * array's device address (hipGetSymbolAddress), later calls reuse it.
 *
 * Arguments, plan, results and errors are those of ssm_scan_fwd (same
 * kernels, bit for bit the same outputs for the same plan), except:
 *   - a plan whose workspace (ssm_scan_fwd_workspace_size) exceeds
 *     MAMBA_NOALLOC_SCRATCH_BYTES returns MAMBA_ERR_WORKSPACE before any
 *     HIP call; a smaller chunk count (a longer chunk_len) may fit;
 *   - every call on one GPU shares that array, so calls that overlap on one
 *     GPU (on different streams or from different threads) race and give
 *     undefined results: callers serialise them, e.g. on one stream. The
 *     array keeps the last call's contents; no call needs it cleared.
 */
int ssm_scan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int dtype,
                         const void* x, const void* delta, const float* A,
                         const void* B, const void* C, const float* D, const void* z,
                         const float* h0, void* y, float* hL,
                         const mamba_scan_options* options, const mamba_scan_plan* plan,
                         hipStream_t stream);

/*
 * Single-token decode update (section "Taken Apart": one token moves the
 * state once). Equivalent to ssm_scan_fwd with seqlen = 1 and h0 = hL = h.
 *
 * h          (batch, dim, dstate) fp32, read and updated in place
 * x, delta   (batch, dim)            required
 * A          (dim, dstate) fp32      required
 * B, C       (batch, dstate)         required
 * D          (dim) fp32              optional
 * z          (batch, dim)            optional
 * y          (batch, dim)            written
 * options    delta bias and activation (may be NULL: none), as for
 *            ssm_scan_fwd
 */
int ssm_state_update(int64_t batch, int64_t dim, int dstate, int dtype, float* h,
                     const void* x, const void* delta, const float* A,
                     const void* B, const void* C, const float* D, const void* z,
                     void* y, const mamba_scan_options* options, hipStream_t stream);

/*
 * Backward pass of ssm_scan_fwd (page "Mamba and State Space Models",
 * section "A Scan on the Chip": the states the backward pass needs are
 * computed again rather than stored). Given the forward call's inputs and
 * the gradients dy at y and dhL at the final state, it writes the gradients
 * of L = sum(dy * y) + sum(dhL * hL) with respect to every input.
 *
 * x, delta, A, B, C, D, z, h0, options   as passed to ssm_scan_fwd
 * dy           (batch, seqlen, dim) I/O dtype     required
 * dhL          (batch, dim, dstate) fp32          optional (NULL: zero)
 * dx, ddelta   (batch, seqlen, dim) I/O dtype     written; ddelta is the
 *                                                 gradient at the delta input
 *                                                 (before the activation when
 *                                                 options apply one)
 * dA           (dim, dstate) fp32                 written (summed over rows)
 * dB, dC       (batch, seqlen, dstate) fp32       written (summed over channels)
 * dD           (dim) fp32                         optional; must be NULL when D is
 * dz           (batch, seqlen, dim) I/O dtype     optional; must be NULL when z is
 * dh0          (batch, dim, dstate) fp32          optional: the gradient at the
 *                                                 initial state (zero start when
 *                                                 h0 is NULL)
 * ddelta_bias  (dim) fp32                         optional; must be NULL when
 *                                                 options carry no delta_bias
 * plan         may be NULL (automatic). `chunk_len` (0: automatic, else a
 *              multiple of 8) cuts the sequence into chunks that run in
 *              parallel; the automatic plan cuts it only when the channel
 *              groups alone hold fewer than two waves per SIMD, into chunks
 *              of at least 64 tokens for about six. `halves` (see
 *              mamba_scan_plan: channel groups run as two 32-channel halves,
 *              dstate 13..16, automatic by the same rule as the forward
 *              scan) needs one chunk: forcing both is MAMBA_ERR_UNSUPPORTED.
 *              state_split, carry and reserved must be 0.
 * workspace    at least the bytes ssm_scan_bwd_workspace_size reports for the
 *              same shape and plan
 *
 * The intermediate states are recomputed from checkpoints every 8 tokens
 * that the call itself computes into the workspace. A chunked sequence first
 * runs every chunk forward from a zero start (chunk 0 from h0), writing its
 * checkpoints and its summary, and summarises every chunk but the first
 * backward from a zero adjoint; both summaries are folded in chunk order
 * into each chunk's entering state and adjoint (the same combine as the
 * forward chunks'), and the walk back adds the entering state, decayed, to
 * each checkpoint it reads, so each chunk's gradients follow from its own
 * tokens. Sums over channels and rows are taken in a fixed order, so
 * results are reproducible bit for bit for a given plan. seqlen == 0 writes
 * zero dA, dD, ddelta_bias and dh0 = dhL. Outputs must not overlap inputs or
 * each other. Errors as for ssm_scan_fwd.
 *
 * ssm_scan_bwd_workspace_size: scratch bytes for the shape and plan; with
 * `resolved` non-NULL it also reports the plan decided (chunk_len: the
 * chunk length, the whole sequence when uncut; halves: the groups split).
 */
int ssm_scan_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int dstate,
                                int dtype, const mamba_scan_plan* plan,
                                mamba_scan_plan* resolved, size_t* bytes);

int ssm_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int dtype,
                 const void* x, const void* delta, const float* A, const void* B,
                 const void* C, const float* D, const void* z, const float* h0,
                 const mamba_scan_options* options, const mamba_scan_plan* plan,
                 const void* dy, const float* dhL,
                 void* dx, void* ddelta, float* dA, float* dB, float* dC, float* dD,
                 void* dz, float* dh0, float* ddelta_bias, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/* Channels per head of the dual form, and the state sizes it provides. */
#define MAMBA_SSD_HEADDIM 64

/*
 * Mamba-2's state space dual form (page "Mamba and State Space Models",
 * section "Mamba-2: Two Algorithms"): A is a number a_h times the identity,
 * shared with the step dt by the 64 channels of a head, so a chunk of the
 * sequence maps input to output through one lower-triangular matrix
 * (entry i, j: C_i . B_j times the decay between) and the chunks are done
 * with matrix products on the matrix cores, passing only the state on.
 * The result is the recurrence, per batch row b, head h, channel p of the
 * head (channel d = h*64 + p) and state n:
 *
 *     h[p,n] <- exp(dt[b,t,h] a_h) h[p,n] + dt[b,t,h] B[b,t,n] x[b,t,d]
 *     y[b,t,d] = (sum_n C[b,t,n] h[p,n] + D[d] x[b,t,d]) * silu(z[b,t,d])
 *
 * x, z, y   (batch, seqlen, nheads*64) bf16      z optional
 * dt        (batch, seqlen, nheads) bf16         positive, or raw with
 *                                                options (delta_bias is then
 *                                                (nheads) fp32, one per head)
 * A         (nheads) fp32                        a_h < 0 (not checked)
 * B, C      (batch, seqlen, dstate) bf16         shared by all heads
 * D         (nheads*64) fp32                     optional
 * h0, hL    (batch, nheads, 64, dstate) fp32     optional; hL may alias h0
 *
 * Requirements: headdim == MAMBA_SSD_HEADDIM, dstate 64 or 128, dtype
 * MAMBA_DTYPE_BF16 (the products run in bf16 with fp32 accumulation),
 * nheads <= 65536; anything else is MAMBA_ERR_UNSUPPORTED. No workspace. Errors and
 * ownership as for ssm_scan_fwd. A NaN or infinite input stays in its channel
 * but, since the chunk products multiply the causal mask's zeros by it, also
 * reaches the earlier outputs of its own 16-token block.
 */
int ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int dstate,
            int dtype, const void* x, const void* dt, const float* A, const void* B,
            const void* C, const float* D, const void* z, const float* h0, void* y, float* hL,
            const mamba_scan_options* options, hipStream_t stream);

/* Widest short convolution the library provides (the pages' width is 4). */
#define MAMBA_CONV_MAX_WIDTH 4

/*
 * Short causal depthwise convolution of the Mamba block over whole
 * sequences (page "Mamba and State Space Models", section "A State of Fixed
 * Size": besides its SSM state each channel keeps the last 4 inputs of a
 * short convolution). The pages give no formula; the library computes, per
 * batch row b, channel d and token t,
 *
 *     pre[b,t,d] = bias[d] + sum_{k=0}^{W-1} weight[d,k] * x[b, t-(W-1)+k, d]
 *     y[b,t,d]   = silu(pre) if silu != 0, else pre
 *
 * each channel filtered on its own and causally: weight[d, W-1] multiplies
 * the current token. Inputs before token 0 come from state_in.
 *
 * x          (batch, seqlen, dim) I/O dtype   required when seqlen > 0
 * weight     (dim, width) fp32                required; 1 <= width <= 4
 * bias       (dim) fp32                       optional (NULL: no bias)
 * state_in   (batch, dim, width) I/O dtype    optional: the last `width`
 *                                             inputs before the sequence,
 *                                             oldest first (NULL: zeros)
 * y          (batch, seqlen, dim) I/O dtype   written
 * state_out  (batch, dim, width) I/O dtype    optional: receives the last
 *                                             `width` inputs of the sequence
 *                                             (reaching into state_in when
 *                                             seqlen < width); may be the
 *                                             same buffer as state_in, but
 *                                             must not partly overlap it
 * The state holds inputs, so it is kept exactly in the I/O dtype. seqlen == 0
 * copies state_in (or zeros) to state_out; batch == 0 or dim == 0 is a
 * no-op. y must not overlap x or the states. Errors as for ssm_scan_fwd;
 * a width outside 1..4 is MAMBA_ERR_UNSUPPORTED.
 */
int causal_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int width, int dtype,
                      const void* x, const float* weight, const float* bias,
                      const void* state_in, void* y, void* state_out, int silu,
                      hipStream_t stream);

/*
 * Decode step of the short convolution: the token's input joins the
 * carried inputs (the oldest leaves) and one output is produced. Equivalent
 * to causal_conv1d_fwd with seqlen = 1 and state_in = state_out = state.
 *
 * state      (batch, dim, width) I/O dtype    read and updated in place
 * x          (batch, dim) I/O dtype           required
 * weight     (dim, width) fp32                required
 * bias       (dim) fp32                       optional
 * y          (batch, dim) I/O dtype           written
 */
int causal_conv1d_update(int64_t batch, int64_t dim, int width, int dtype, void* state,
                         const void* x, const float* weight, const float* bias, void* y,
                         int silu, hipStream_t stream);

/* Static, human-readable name of a mamba_status value. */
const char* mamba_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SCAN_H */
