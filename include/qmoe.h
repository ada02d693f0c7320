/*
 * qmoe.h - C ABI of one tensor-parallel rank's routed-MoE layer call on an
 * MI355X (gfx950) GPU.
 *
 * The call (pages: "IQ2R: load GLM-5.3 packed MoE checkpoints with TP
 * slicing" and "[HIP] IQ2R: GLM-5.3 packed MoE path for TP4/TP8 on gfx950",
 * Summary sections; "glm53: FP8 mid hand-off, early split rows, per-row
 * up/gate jobs, ...", Modifications table) computes, for M tokens:
 *
 *   1. top-k routing of fp32 router logits (ties go to the lower expert id),
 *      weights = sigmoid scores renormalized over the k slots x routed scaling
 *   2. a stable sort of the M*k (token, slot) entries by expert
 *   3. x (bf16) -> MXFP4 once per token (E2M1, one E8M0 scale per 32)
 *   4. gate/up GEMM on MXFP4 expert weights, h = SiLU(gate) * up
 *   5. h -> FP8 E4M3 once per 128-element block, with an fp32 scale (or,
 *      with moe_plan_set_mid_format, MXFP4 per 32 for the stock MXFP4 arm)
 *   6. down GEMM on MXFP4 expert weights
 *   7. out (bf16) = sum over slots of weight * down output (+ shared expert)
 *   8. optional block-FP8 shared expert (128x128 weight scales), weight 1
 *
 * Conventions for every entry point:
 *   - All tensors are dense, row-major (the weights moe_pack_w13 and
 *     moe_pack_w2 write excepted), 16-byte aligned device pointers on
 *     the plan's device. The caller owns every buffer (inputs, weights,
 *     output, workspace); the library never allocates device memory and
 *     never synchronizes a stream. `stream` is a hipStream_t (NULL = the
 *     default stream). All GPU work of a call is enqueued on that stream in
 *     order, so a call may be captured into a HIP graph.
 *   - Arguments are validated before anything is enqueued; on a validation
 *     error nothing is launched and nothing is written.
 *   - MXFP4 bytes hold two E2M1 codes, element 2i in the low nibble.
 *   - One plan, with its workspace, serves one stream at a time.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null / misaligned pointer, bad size, k > E, M > plan maximum */
  MOE_ERR_UNSUPPORTED = 2,  /* shape outside what the kernels handle (see moe_plan_create) */
  MOE_ERR_WORKSPACE = 3,    /* workspace missing, too small or misaligned */
  MOE_ERR_DEVICE = 4,       /* no usable gfx950 device, or pointers on another device */
  MOE_ERR_HIP = 5           /* the HIP runtime reported an error while enqueueing */
} moe_status;

/* One rank's shape. M is the largest token count a call on this plan may use. */
typedef struct {
  int64_t M;              /* max tokens per call, >= 0 */
  int64_t H;              /* hidden size, multiple of 512 */
  int64_t E;              /* routed experts, 1..1024 */
  int64_t I;              /* intermediate size per rank: 128, 256, 384 or 512 */
  int64_t top_k;          /* 1..min(E, 16) */
  float routed_scaling;   /* routing weights of a token sum to this (finite, > 0) */
  int64_t shared_I;       /* shared-expert intermediate size (multiple of 128), 0 = none */
} moe_shape;

typedef struct moe_plan moe_plan; /* opaque; host memory only */

/* Byte offsets into the workspace of the intermediates a call leaves behind
 * (valid until the next call on the plan). Layouts, with n = M * top_k:
 *   topk_ids     int32 [M, k]       expert of slot j of token t
 *   topk_w       fp32  [M, k]       routing weight (includes routed_scaling)
 *   count        int32 [E]          entries per expert
 *   offset       int32 [E + 1]      exclusive prefix of count
 *   sorted_entry int32 [n]          entries t*k+j grouped by expert, t ascending
 *   xq           u8    [M, H/2]     x as E2M1 codes (MXFP4)
 *   xs           u8    [M, H/32]    x's E8M0 scales
 *   midq         u8    [n, I]       E4M3 mid, rows in sorted order
 *   mids         fp32  [n, I/128]   mid block scales, rows in sorted order
 *   y            fp32  [n, H]       unweighted down output, row = entry t*k+j;
 *                                   written only by calls with M > 16 (up to
 *                                   16 tokens the combine runs in the down
 *                                   launch and slot results stay on chip)
 *   sh_xq/sh_xs  i8 [M, H/128, 3, 128] / fp32 [H/128, M]  shared expert x
 *   sh_hq/sh_hs  i8 [M, Is/128, 3, 128] / fp32 [Is/128, M] shared expert mid
 *                                   (E4M3 values v as digit rows: for each
 *                                   128-block, three planes of 128 int8 d0,
 *                                   d1, d2 with v * 2^9 = d0 + 2^7 d1 +
 *                                   2^14 d2, all of v's sign; rows past M,
 *                                   up to a multiple of 128, are padding;
 *                                   scales K-block major: block b of token t
 *                                   at b * M + t)
 *   sh_y         fp32  [M, H]       shared expert output
 * A call of at most 16 tokens (and 512 slots) with the E4M3 mid and
 * shared_I <= 512 runs the shared expert inside the routed launches: its
 * sh_xq and sh_hq then hold plain E4M3 codes, u8 [M, H] and u8 [M, Is]
 * (scales as above), and sh_y is not written (each down workgroup adds its
 * columns of the shared output into the combine). Offsets of absent parts
 * (no shared expert) are 0. */
typedef struct {
  size_t total_bytes;
  size_t topk_ids, topk_w, count, offset, sorted_entry;
  size_t xq, xs, midq, mids, y;
  size_t sh_xq, sh_xs, sh_hq, sh_hs, sh_y;
} moe_ws_layout;

/* Create a host-side plan for `shape` on the current HIP device.
 * Returns MOE_ERR_INVALID_ARG for null arguments, negative or zero sizes,
 * top_k > E or a non-positive routed_scaling; MOE_ERR_UNSUPPORTED for
 * H % 512 != 0, I not in {128, 256, 384, 512}, E > 1024, top_k > 16,
 * shared_I % 128 != 0 or shared_I > 2048, M > 2^20, H > 65536 or
 * M * H / 2 > 2^31 - 1 (x's FP4 codes are addressed with 32-bit byte
 * offsets); MOE_ERR_DEVICE when the
 * current HIP device cannot be queried or is not a gfx950. Creating a plan
 * enqueues no GPU work. */
moe_status moe_plan_create(const moe_shape* shape, moe_plan** out);

/* Workspace bytes a plan of this shape needs, computed on the host alone
 * (no device is queried). Same validation as moe_plan_create. */
moe_status moe_shape_workspace_bytes(const moe_shape* shape, size_t* bytes);

/* Free the plan (not the caller's workspace). NULL is accepted. */
void moe_plan_destroy(moe_plan* plan);

/* Bytes of device workspace the plan needs (multiple of 256). */
size_t moe_plan_workspace_bytes(const moe_plan* plan);

/* Offsets of the intermediates inside the workspace. */
moe_status moe_plan_layout(const moe_plan* plan, moe_ws_layout* out);

/* Bind a caller-owned device workspace (256-byte aligned, at least
 * moe_plan_workspace_bytes) to the plan and enqueue on `stream` the one-time
 * initialisation of its synchronisation counters. The workspace must not be
 * written by the caller afterwards. MOE_ERR_WORKSPACE if it is too small or
 * misaligned, MOE_ERR_DEVICE if it lives on another device. */
moe_status moe_plan_set_workspace(moe_plan* plan, void* workspace, size_t bytes, void* stream);

/* Bytes of the device buffer moe_plan_set_shared packs the shared expert's
 * weights into: 12 * shared_I * H (0 for a plan without a shared expert). */
size_t moe_plan_shared_pack_bytes(const moe_plan* plan);

/* Bind the block-FP8 shared expert (required iff shape.shared_I > 0; "IQ2R:
 * load GLM-5.3 packed MoE checkpoints with TP slicing", Summary: the shared
 * experts keep the base model's block-FP8 configuration). Inputs, row-major:
 *   ws13 u8 (E4M3) [2*Is, H]  rows [0, Is) gate, [Is, 2*Is) up
 *   ss13 fp32 [2*Is/128, H/128]  one scale per 128x128 block
 *   ws2  u8 (E4M3) [H, Is];  ss2 fp32 [H/128, Is/128]
 * `packed` is a caller-owned device buffer of at least
 * moe_plan_shared_pack_bytes(plan) bytes, not overlapping the inputs; the
 * call enqueues on `stream` the one-time rewrite of ws13 and ws2 into it
 * (each E4M3 value as three int8 digits of its value times 2^9, the
 * operands of the exact int8-MFMA GEMMs; nothing is rounded), followed by
 * a copy of the E4M3 codes themselves (read by calls that run the shared
 * expert inside the routed launches). The plan
 * keeps `packed`, ss13 and ss2 (not copied: they must stay valid while the
 * plan is used); ws13 and ws2 are read only by the enqueued rewrite.
 * MOE_ERR_INVALID_ARG for null or misaligned pointers, a plan without a
 * shared expert, a short or overlapping `packed`; MOE_ERR_DEVICE for
 * pointers on another device than the plan's. */
moe_status moe_plan_set_shared(moe_plan* plan, const void* ws13, const float* ss13, const void* ws2,
                               const float* ss2, void* packed, size_t packed_bytes, void* stream);

/* Format of the mid hand-off between gate/up and down. MOE_MID_E4M3 (the
 * default): one E4M3 code per element and an fp32 scale per 128 ("glm53: FP8
 * mid hand-off, early split rows, ...", Modifications table, row "mid as FP8
 * once"), down on exact bf16 products. MOE_MID_MXFP4: the comparison arm the
 * pages time against IQ2R, stock experts quantized online to MXFP4 ("IQ2R:
 * load GLM-5.3 packed MoE checkpoints with TP slicing", Results (MXFP4 vs
 * IQ2R)), read as FP4 activations in both GEMMs: mid per 32 as E2M1 codes
 * with an E8M0 scale (the rule x takes), down on the scaled FP4 MFMA. With
 * MXFP4, moe_forward's w2 and s2 are the packed ones of moe_pack_w2, the
 * workspace's midq holds [n, I/2] codes (element 2i in the low nibble) and
 * mids [n, I/32] scale bytes, rows in sorted order, and y is written for
 * every M. */
typedef enum { MOE_MID_E4M3 = 0, MOE_MID_MXFP4 = 1 } moe_mid_format;

/* Fuse a shared expert as the last expert and the last slot ("[HIP] IQ2R:
 * GLM-5.3 packed MoE path for TP4/TP8 on gfx950", Summary: 256 routed
 * experts plus the shared expert as expert 256, top-9). With on = 1 the
 * plan's expert E-1 is the shared expert, given in the routed experts'
 * format as the last expert of w13/s13/w2/s2; slots 0..top_k-2 of every
 * token are routed over the first E-1 logits (the last logits column is not
 * read, weights renormalized over those slots) and slot top_k-1 is expert
 * E-1 with weight 1. MOE_ERR_INVALID_ARG for a NULL plan, on not 0 or 1,
 * top_k < 2, or a plan with a block-FP8 shared expert (shape.shared_I > 0).
 * Host-only; applies to later calls. */
moe_status moe_plan_set_shared_slot(moe_plan* plan, int on);

/* Select the mid format for the plan's later calls. MOE_ERR_INVALID_ARG for
 * a NULL plan or an unknown format. Host-only. */
moe_status moe_plan_set_mid_format(moe_plan* plan, int format);

/* Layout of the weights a call receives, declared by the caller once they
 * are in place (the MoE method of "IQ2R: load GLM-5.3 packed MoE checkpoints
 * with TP slicing", Summary, allocates packed expert tensors when the
 * checkpoint is loaded). Flags: MOE_LAYOUT_W13_PACKED, w13/s13 written by
 * moe_pack_w13; MOE_LAYOUT_W2_PACKED, w2/s2 written by moe_pack_w2. The
 * kernels read gate/up weights only packed, and down weights packed exactly
 * when the mid format is MOE_MID_MXFP4, so moe_forward and
 * moe_forward_noalloc return MOE_ERR_UNSUPPORTED, before anything is
 * enqueued, unless the plan's declared layout is MOE_LAYOUT_W13_PACKED with
 * MOE_LAYOUT_W2_PACKED matching the mid format (a new plan declares
 * nothing: a caller passing row-major weights is refused, not served with
 * a wrong result). MOE_ERR_INVALID_ARG for a NULL plan or unknown flags.
 * Host-only; applies to later calls. */
typedef enum { MOE_LAYOUT_W13_PACKED = 1, MOE_LAYOUT_W2_PACKED = 2 } moe_weight_layout;
moe_status moe_plan_set_weight_layout(moe_plan* plan, unsigned layout);

/* Rewrite the routed experts' gate/up weights into the packed layout that
 * moe_forward reads, once, when the weights are loaded (the MoE method of
 * "IQ2R: load GLM-5.3 packed MoE checkpoints with TP slicing", Summary,
 * allocates packed expert tensors at load time). Inputs, row-major:
 *   w13  u8 MXFP4 [E, 2I, H/2]   rows [0, I) gate, [I, 2I) up, along H
 *   s13  u8 E8M0  [E, 2I, H/32]  one scale per 32 elements
 * Outputs, caller-allocated device buffers of the same sizes:
 *   w13_packed [E*2I/16][H/128][4][16][16]: bytes 16*g .. 16*g + 15 of
 *     K-step ks (bytes 64*ks .. 64*ks + 63 of a row) of row 16*rb + r at
 *     (((rb * H/128 + ks) * 4 + g) * 16 + r) * 16
 *   s13_packed [E*2I/16][H/512][4][16][4]: byte j of the dword at
 *     ((rb * H/512 + kq) * 4 + g) * 16 + r holds the scale of MX block
 *     16*kq + 4*j + g of row 16*rb + r
 * (rb runs over the E*2I/16 blocks of 16 rows, experts one after another).
 * A byte permutation: nothing is rounded. All four pointers on one device,
 * 16-byte aligned, outputs not overlapping each other or the inputs.
 * Enqueued on `stream`; nothing is allocated. MOE_ERR_INVALID_ARG for null,
 * misaligned or overlapping pointers or non-positive sizes;
 * MOE_ERR_UNSUPPORTED for the shapes moe_plan_create rejects (H % 512 != 0,
 * H > 65536, I not in {128, 256, 384, 512}, E > 1024); MOE_ERR_DEVICE for
 * host pointers or pointers on different devices. */
moe_status moe_pack_w13(const void* w13, const void* s13, int64_t E, int64_t I, int64_t H,
                        void* w13_packed, void* s13_packed, void* stream);

/* Rewrite the routed experts' down weights for the MXFP4-mid down
 * (MOE_MID_MXFP4 only; the E4M3 mid reads them row-major), once, at load
 * time. Inputs, row-major: w2 u8 MXFP4 [E, H, I/2] along I, s2 u8 E8M0
 * [E, H, I/32]. Outputs, caller-allocated device buffers:
 *   w2_packed [E*H/16][I/128][4][16][16] (the size of w2): bytes 16*g ..
 *     16*g + 15 of K-step ks of row 16*rb + r at
 *     (((rb * I/128 + ks) * 4 + g) * 16 + r) * 16
 *   s2_packed [E*H/16][4][16][4] (E*H*16 bytes): byte ks of the dword at
 *     (rb * 4 + g) * 16 + r holds the scale of MX block 4*ks + g of row
 *     16*rb + r for ks < I/128, zero above
 * (rows are the E*H output columns, experts one after another). A byte
 * permutation: nothing is rounded. Validation and errors as moe_pack_w13. */
moe_status moe_pack_w2(const void* w2, const void* s2, int64_t E, int64_t I, int64_t H,
                       void* w2_packed, void* s2_packed, void* stream);

/* The routed-MoE call on M tokens (0 <= M <= shape.M; M = 0 enqueues nothing):
 *   x      bf16 [M, H]
 *   logits fp32 [M, E]     (finite or -inf)
 *   w13    gate/up weights in the packed layout of moe_pack_w13 (the
 *          MXFP4 [E, 2I, H/2] rows [0, I) gate, [I, 2I) up, along H),
 *          declared with moe_plan_set_weight_layout
 *   s13    their E8M0 scales, packed by moe_pack_w13 ([E, 2I, H/32])
 *   w2     u8 MXFP4 [E, H, I/2]    along I, row-major (packed by
 *          moe_pack_w2 when the plan's mid format is MOE_MID_MXFP4)
 *   s2     u8 E8M0  [E, H, I/32]   (packed likewise)
 *   out    bf16 [M, H]  fully overwritten; must not alias any input
 * Returns after enqueueing; faults inside kernels surface at the caller's
 * next synchronisation. MOE_ERR_WORKSPACE if no workspace is bound,
 * MOE_ERR_INVALID_ARG if the shared expert is required but not bound,
 * MOE_ERR_UNSUPPORTED if the declared weight layout is not the one read.
 * MOE_ERR_HIP when a launch fails once the call has started enqueueing: the
 * launches already enqueued stay (and may write the workspace and `out`),
 * and the workspace is unbound, so later calls return MOE_ERR_WORKSPACE
 * until moe_plan_set_workspace binds (and re-initialises) one again. */
moe_status moe_forward(moe_plan* plan, int64_t M, const void* x, const float* logits,
                       const void* w13, const void* s13, const void* w2, const void* s2,
                       void* out, void* stream);

/* Tensor-parallel partial-sum exchange ("glm53: FP8 mid hand-off, early
 * split rows, per-row up/gate jobs, ...", Accuracy Tests: a rank's peers'
 * partial sums arrive tagged with the launch's epoch, and a one-GPU check
 * runs rank 0 alone with zero peer partials and its pushes going to scratch
 * sinks). With an exchange set on the plan, a call's combine keeps the
 * rank's float64 partial (the slot-order sum before its bf16 rounding) in
 * the rank's own inbox slot, then an epilogue launch pushes it to every
 * peer, waits for the peers' partials, adds all tp partials in float64 in
 * rank order 0..tp-1 and rounds once to bf16 into `out`: every rank forms
 * the same bits. All buffers are caller-owned device memory; M below is the
 * plan's maximum M, slots are indexed by rank:
 *   inbox       fp64 [tp][M][H]: slot r receives rank r's partial (the
 *               rank's own slot is written by the combine)
 *   inbox_tags  u32 [tp][M][H/512]: tag of each 512-column chunk of a slot,
 *               written (by the sender, after the chunk) as the epoch
 *   push[p], push_tags[p]  for p != rank: where this rank's partial and its
 *               tags go for peer p ([M][H] and [M][H/512]; peer p's inbox
 *               slot `rank` in a real group, scratch sinks in a loopback);
 *               entries p >= tp and p == rank are ignored
 *   epoch       nonzero tag of this call's partials (a new one every call)
 *   spin_limit  polls of a peer's tag before the wait gives up: the chunk
 *               is then summed with whatever its slot holds and *status gets
 *               bit 0 set (the call never hangs)
 *   status      u32: set by the epilogue on a failed wait, never cleared */
#define MOE_TP_MAX 8
typedef struct {
  int32_t tp;            /* ranks in the group, 1..MOE_TP_MAX */
  int32_t rank;          /* this rank, 0..tp-1 */
  uint32_t epoch;
  int32_t spin_limit;    /* > 0 */
  double* inbox;
  uint32_t* inbox_tags;
  double* push[MOE_TP_MAX];
  uint32_t* push_tags[MOE_TP_MAX];
  uint32_t* status;
} moe_tp_exchange;

/* Turn the exchange on for later calls (copied into the plan: set a new
 * epoch before every call), or off with NULL. MOE_ERR_INVALID_ARG for a NULL
 * plan, tp or rank out of range, a zero epoch, spin_limit <= 0, or a NULL or
 * misaligned (16 bytes; tags 4) pointer that the group needs;
 * MOE_ERR_UNSUPPORTED for H % 512 != 0 (always true of a valid plan) or the
 * MXFP4 mid (its combine is not split); MOE_ERR_DEVICE for pointers on
 * another device. Host-only. */
moe_status moe_plan_set_tp_exchange(moe_plan* plan, const moe_tp_exchange* x);

/* Bytes of the device scratch moe_forward_noalloc runs on: 64 MiB, one copy
 * per device the library runs on, held until the process ends. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* moe_forward for callers that cannot allocate device memory or bind a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same call, the same kernels and results, with
 * the library's static per-device scratch of MOE_NOALLOC_SCRATCH_BYTES as
 * the workspace instead of the plan's (which is neither needed nor touched;
 * the intermediates of moe_plan_layout are then in that scratch). Allocates
 * nothing and calls no allocating routine. The caller still passes inputs
 * and outputs as for moe_forward, with the same checks.
 * MOE_ERR_UNSUPPORTED when the plan's workspace (moe_plan_workspace_bytes,
 * set by its shape's maximum M) exceeds MOE_NOALLOC_SCRATCH_BYTES, before
 * anything is enqueued; MOE_ERR_HIP when the scratch's address cannot be
 * found or a launch fails. Every call on a device shares that device's
 * scratch, which keeps the last call's contents: calls that may overlap on
 * one device (other streams, other host threads) race and must not be
 * issued; the call clears what it needs zeroed itself. */
moe_status moe_forward_noalloc(moe_plan* plan, int64_t M, const void* x, const float* logits,
                               const void* w13, const void* s13, const void* w2, const void* s2,
                               void* out, void* stream);

/* Profiling aid: when `events` is non-NULL, moe_forward brackets stage i
 * with events[2i] (start of its first kernel) and events[2i+1] (end of its
 * last kernel), hipEvent_t handles, so hipEventElapsedTime(events[2i],
 * events[2i+1]) is the stage's execution time. A stage folded into another
 * one for small M records an empty interval. `n` must be
 * 2 * moe_stage_count(). NULL disables. */
moe_status moe_plan_set_stage_events(moe_plan* plan, void* const* events, int n);

/* Profiling aid: when `start` and `stop` are non-NULL hipEvent_t handles,
 * moe_forward records `start` as its first kernel begins and `stop` as its
 * last kernel ends, so hipEventElapsedTime(start, stop) is the call's device
 * time without the host's launch latency. Replaces the stage events above
 * (and they replace these); NULL, NULL disables. Both or neither must be
 * NULL, else MOE_ERR_INVALID_ARG. */
moe_status moe_plan_set_call_events(moe_plan* plan, void* start, void* stop);

/* Number and names of the launch stages of a call (for the events above). */
int moe_stage_count(void);
const char* moe_stage_name(int i);

/* Kernels that stage `stage` launches for a call of M tokens on this plan
 * with its current mid format (0 when the stage is folded into another
 * one), or -1 for bad arguments (M outside [0, the plan's M], an unknown
 * stage). */
int moe_plan_stage_launches(const moe_plan* plan, int64_t M, int stage);

/* Static text for a status code. */
const char* moe_status_str(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
