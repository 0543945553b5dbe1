/*
 * moe.h -- C ABI of the routed mixture-of-experts layer for small-row decode
 * and speculative-verify steps (rows = 1..16), built for AMD Instinct MI355X
 * (gfx950) as libmoe.so.
 *
 * What is computed (sources are cited by page title and section):
 *
 *   "Function forward_moe" rustdoc, signature and summary: one routed MoE
 *   site maps x[rows, h] to out[rows, h] given weights, a workspace and a
 *   stream.  On one GPU ``out`` holds the full result (the page leaves a
 *   partial sum only when experts or the shared expert are split over ranks).
 *
 *   metrale_model_layers/layers/moe/forward_token_major.rs,
 *   MoeLayer::forward_token_major_decode: router GEMM over the rows; batched
 *   top-k (softmax with norm_topk_prob, or sigmoid with a per-expert
 *   correction bias, norm_topk_prob and routed_scaling_factor); expert
 *   gate+up; silu(gate)*up and down; weighted sum plus the blend of the
 *   shared expert gated by the input and shared_expert_gate.weight.  Experts
 *   are untransposed NVFP4 matrices reached through device pointer tables of
 *   packed codes, scales and scale2 values.
 *
 *   "Function forward_moe" rustdoc, "RETRACTED (2026-08-29)" and
 *   "WIDENED (2026-08-31)" notes: the selected ids are deduplicated in one
 *   block by a pairwise scan (no sort), and each expert of the union is
 *   swept once for all rows that chose it.  The pages' block holds
 *   top_k*rows <= 64 ids (8 rows x 8); here the same scan runs over up to
 *   two 64-slot tiles, so one call takes up to 16 rows and 128 ids.
 *   SHARED-expert note: the shared expert runs once over all rows.
 *
 * Per row r:
 *   L[r,e]   = sum_t x[r,t] * router_w[e,t]                     (fp32 result;
 *              router_w dense fp32, or the NVFP4 router_nvfp4 decoded exactly)
 *   softmax: ids = top_k of L[r,:]; w = softmax weights of those ids,
 *            renormalised over the k ids when norm_topk_prob.
 *   sigmoid: s = sigmoid(L); ids = top_k of fp32(fp32(s) + bias) (s rounded
 *            to fp32, then an fp32 add);
 *            w = s[ids] (renormalised when norm_topk_prob) * routed_scaling_factor.
 *   ids within a row are ordered by descending key, equal keys by lower id.
 *   FFN_e(x) = W_down[e] @ (silu(W_gate[e] @ x) * (W_up[e] @ x))
 *   out[r]   = bf16( sum_j w[r,j] * FFN_{ids[r,j]}(x_r)
 *                    + sigmoid(x_r . shared_expert_gate) * FFN_shared(x_r) )
 *            (gate 1 when shared_expert_gate is NULL)
 *
 * NVFP4 matrix [n, k] ("untransposed": k contiguous):
 *   packed  uint8 [n, k/2]   two E2M1 codes per byte, even column in the low nibble
 *   scales  uint8 [n, k/16]  OCP E4M3FN scale for each 16 consecutive columns
 *   scale2  fp32             per-tensor scale
 *   W[i,t] = e2m1(code[i,t]) * e4m3(scales[i, t/16]) * scale2
 * gate/up are [I, h], down is [h, I] (I = moe_inter or shared_inter).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are device pointers the caller allocates and owns.
 *     The library keeps no pointer after a call returns and allocates no
 *     device or host memory on any call.
 *   - Calls validate on the host, enqueue kernels on ``stream`` (a
 *     hipStream_t passed as void*, NULL = default stream) and return.  There
 *     is no host synchronisation, no device-to-host copy and no host branch on
 *     the routing, so every call can be captured into a HIP graph.  Results
 *     are visible once the caller synchronises with the stream.
 *   - Every argument error is reported before any HIP call.  No exception
 *     crosses the ABI.  A non-OK status leaves a message for moe_last_error().
 *   - One workspace serves one in-flight call.  Calls that share a workspace
 *     must be ordered on one stream.
 *   - Ids outside [0, num_experts) or repeated ids within a row, passed to
 *     moe_union, are outside the contract (results are unspecified; the
 *     kernels still read and write only in bounds of the documented buffers).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* bad pointer, size, alignment, overlap or enum */
  MOE_ERR_UNSUPPORTED = 2, /* a valid layer this library does not serve     */
  MOE_ERR_WORKSPACE = 3,   /* ws_bytes < moe_workspace_bytes(cfg)            */
  MOE_ERR_DEVICE = 4       /* a HIP launch or runtime error                  */
} moe_status;

enum {
  MOE_ROUTE_SOFTMAX = 0,      /* softmax top-k, optional renormalisation        */
  MOE_ROUTE_SIGMOID_BIAS = 1, /* sigmoid + correction bias, routed_scaling_factor */
  MOE_MAX_ROWS = 16,          /* rows per call                                   */
  MOE_MAX_IDS = 128,          /* top_k * rows, two tiles of MOE_BLOCK_IDS         */
  MOE_BLOCK_IDS = 64,         /* the one-block union of the "RETRACTED (2026-08-29)"
                                 and "WIDENED (2026-08-31)" notes: 8 rows x 8    */
  MOE_MAX_CHUNK_ROWS = 36,    /* rows * ceil(hidden / 2048) a call stages in LDS */
  MOE_MAX_EXPERTS = 1024,     /* design cap on num_experts                       */
  MOE_MAX_DIM = 8192,         /* cap on hidden                                   */
  MOE_MAX_INTER = 4096,       /* cap on moe_inter and shared_inter               */
  MOE_DIM_ALIGN = 32,         /* hidden, moe_inter, shared_inter multiple of 32  */
  MOE_STATIC_SCRATCH_BYTES = 8 << 20 /* moe_forward_static's workspace, per GPU   */
};

/* Layer configuration (Glm5NextMlpConfig subset used by the routed path). */
typedef struct moe_config {
  int32_t hidden;               /* h                                            */
  int32_t num_experts;          /* E, 1..MOE_MAX_EXPERTS                        */
  int32_t top_k;                /* k, 1..E, and k * rows <= MOE_MAX_IDS         */
  int32_t moe_inter;            /* I of a routed expert                          */
  int32_t shared_inter;         /* Is of the shared expert                       */
  int32_t route_kind;           /* MOE_ROUTE_SOFTMAX or MOE_ROUTE_SIGMOID_BIAS   */
  int32_t norm_topk_prob;       /* 0 or 1                                        */
  float routed_scaling_factor;  /* sigmoid routing only; softmax ignores it      */
} moe_config;

/* One NVFP4 matrix (layout above).  Both pointers 16-byte aligned. */
typedef struct moe_nvfp4 {
  const uint8_t* packed;
  const uint8_t* scales;
  float scale2;
} moe_nvfp4;

/* One projection of every routed expert, as device arrays indexed by expert
 * id: packed[e] and scales[e] are device pointers (16-byte aligned) to
 * expert e's matrix, scale2[e] its fp32 per-tensor scale.  The three arrays
 * themselves live in device memory (forward_token_major.rs passes
 * packed_ptrs, scale_ptrs and scale2_vals the same way). */
typedef struct moe_expert_table {
  const uint8_t* const* packed; /* device array [E] of device pointers */
  const uint8_t* const* scales; /* device array [E] of device pointers */
  const float* scale2;          /* device array [E]                    */
} moe_expert_table;

typedef struct moe_weights {
  const float* router_w;           /* [E, h] fp32, row-major; NULL: router_nvfp4 */
  const float* correction_bias;    /* [E] fp32 for SIGMOID_BIAS, NULL otherwise  */
  moe_expert_table gate;           /* [I, h] per expert                          */
  moe_expert_table up;             /* [I, h] per expert                          */
  moe_expert_table down;           /* [h, I] per expert                          */
  moe_nvfp4 shared_gate;           /* [Is, h]                                    */
  moe_nvfp4 shared_up;             /* [Is, h]                                    */
  moe_nvfp4 shared_down;           /* [h, Is]                                    */
  const float* shared_expert_gate; /* [h] fp32: gate = sigmoid(x . this); NULL:
                                      the shared expert is added ungated (gate 1),
                                      as forward_token_major.rs does with
                                      residual_add when the gate weight is null */
  moe_nvfp4 router_nvfp4;          /* [E, h] NVFP4 router, used when router_w is
                                      NULL (forward_ep.rs and
                                      forward_token_major.rs run the gate
                                      projection as an NVFP4 GEMV / GEMM); its
                                      packed and scales must be NULL when
                                      router_w is set */
} moe_weights;

/* Byte offsets of the intermediates moe_forward leaves in the workspace.
 * The layout depends on the config only (sized for MOE_MAX_ROWS rows).
 * Offsets are multiples of 256.  The workspace needs no initialisation: every
 * call writes what it reads.  Calls sharing one workspace must not overlap in
 * time (same stream, or ordered by events).
 *
 * Expert activations and outputs are stored by (row, selected expert) pair:
 * pair t = r*k + j holds row r's j-th routed expert, pair rows*k + r row r's
 * shared expert. */
typedef struct moe_ws_layout {
  size_t logits;        /* float  [MOE_MAX_ROWS][E]   router logits (row stride E)    */
  size_t score;         /* double [MOE_MAX_ROWS][E]   sigmoid(logit) for sigmoid routing */
  size_t gamma;         /* float  [MOE_MAX_ROWS]      sigmoid(x_r . shared gate)      */
  size_t topk_ids;      /* int32  [MOE_MAX_ROWS][k]   (row stride k)                  */
  size_t topk_w;        /* float  [MOE_MAX_ROWS][k]                                   */
  size_t union_ids;     /* int32  [MOE_MAX_IDS]       first-occurrence order          */
  size_t union_count;   /* int32  [1]                 U                               */
  size_t slot_to_union; /* int32  [MOE_MAX_IDS]       slot t = r*k + j -> union index */
  size_t row_mask;      /* uint32 [MOE_MAX_IDS]       bit r: row r chose union expert */
  size_t slot_info;     /* internal per-union-slot weight pointers                    */
  size_t segments;      /* internal down-sweep work table                             */
  size_t act;           /* bf16   [MOE_MAX_IDS+MOE_MAX_ROWS][Imax] silu(g)*u by pair,
                           Imax = max(I, Is); pairs rows*(k+1) and up unused          */
  size_t y;             /* float  [MOE_MAX_IDS+MOE_MAX_ROWS][h] expert outputs by pair */
  size_t total;         /* bytes needed                                               */
} moe_ws_layout;

/* Workspace bytes for ``cfg`` (any rows up to MOE_MAX_ROWS); 0 if cfg is
 * invalid.  The workspace may hold anything before a call. */
size_t moe_workspace_bytes(const moe_config* cfg);

/* Fill ``out`` with the workspace layout of ``cfg``. */
moe_status moe_workspace_layout(const moe_config* cfg, moe_ws_layout* out);

/* Router and top-k routing (forward_token_major.rs: router GEMM, then
 * moe_topk_sigmoid_batched or moe_topk_softmax_batched; forward_ep.rs: the
 * one-row GEMV and moe_topk_softmax).
 *   x_bf16    [rows, h] bf16 bits, 16-byte aligned
 *   rows      1 .. MOE_MAX_ROWS with top_k * rows <= MOE_MAX_IDS, at any
 *             hidden size (the router stages no x; moe_forward may take fewer)
 *   topk_ids  [rows, k] int32 out, ordered by descending key, ties by lower id
 *   topk_w    [rows, k] fp32 out
 * Also leaves logits and gamma in the workspace. */
moe_status moe_route(const moe_config* cfg, const moe_weights* w, const uint16_t* x_bf16,
                     int32_t rows, int32_t* topk_ids, float* topk_w,
                     void* ws, size_t ws_bytes, void* stream);

/* Union of the experts selected by ``rows`` rows ("Function forward_moe"
 * rustdoc, "RETRACTED (2026-08-29)" note: one block, pairwise scan, no sort).
 * Up to MOE_BLOCK_IDS ids this is that one-block union; up to MOE_MAX_IDS the
 * same scan runs over two tiles of MOE_BLOCK_IDS slots and the second tile's
 * union positions continue the first's (the order stays first occurrence in
 * row-major slot order).
 *   topk_ids       [rows, top_k] int32 in, each row's ids distinct, in [0, num_experts)
 *   union_ids      [MOE_MAX_IDS] out, first occurrence in row-major slot order
 *   union_count    [1] out, U
 *   slot_to_union  [rows*top_k] out, union position of slot t = r*top_k + j
 *   row_mask       [MOE_MAX_IDS] out, bit r set when row r chose union expert u;
 *                  may be NULL
 * Entries of union_ids and row_mask at positions >= U are left untouched. */
moe_status moe_union(const int32_t* topk_ids, int32_t rows, int32_t top_k, int32_t num_experts,
                     int32_t* union_ids, int32_t* union_count, int32_t* slot_to_union,
                     uint32_t* row_mask, void* stream);

/* moe_union restricted to the experts in [expert_lo, expert_hi): one GPU's
 * share under expert parallelism (forward_ep.rs splits the selected ids into
 * local and remote ones by local_expert_range and build_ep_routing_table).
 * Slots whose id is outside the range get slot_to_union = -1 and are not in
 * the union; the others form it as moe_union does.  Arguments and refusals
 * as moe_union, plus 0 <= expert_lo <= expert_hi <= num_experts. */
moe_status moe_union_local(const int32_t* topk_ids, int32_t rows, int32_t top_k, int32_t num_experts,
                           int32_t expert_lo, int32_t expert_hi, int32_t* union_ids, int32_t* union_count,
                           int32_t* slot_to_union, uint32_t* row_mask, void* stream);

/* The whole layer: x[rows, h] bf16 -> out[rows, h] bf16 (overwritten, not
 * accumulated).  x and out 16-byte aligned and not overlapping.  Leaves every
 * intermediate of moe_ws_layout in the workspace.  Each row's output depends
 * on that row's input alone: a call with R rows writes, for every row, the
 * same bytes as a one-row call with that row.  rows <= MOE_MAX_ROWS with
 * top_k * rows <= MOE_MAX_IDS; rows * ceil(hidden / 2048) > MOE_MAX_CHUNK_ROWS
 * is refused with MOE_ERR_UNSUPPORTED (the sweep keeps every row of x in LDS;
 * moe_forward_prefill serves longer batches). */
moe_status moe_forward(const moe_config* cfg, const moe_weights* w, const uint16_t* x_bf16,
                       uint16_t* out_bf16, int32_t rows, void* ws, size_t ws_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * workspace is the library's own array of MOE_STATIC_SCRATCH_BYTES in each
 * GPU's memory, held from the first call on that GPU until the process ends.
 * Nothing else differs from moe_forward: same arguments (no workspace),
 * refusals and output bytes.  The call allocates nothing.  Refused with
 * MOE_ERR_UNSUPPORTED, before any HIP call, when moe_workspace_bytes(cfg)
 * exceeds MOE_STATIC_SCRATCH_BYTES.  Every call on one GPU shares that GPU's
 * array, which keeps the last call's intermediates: calls that overlap in
 * time on one GPU (other streams, other threads) race and give undefined
 * results; order them on one stream. */
moe_status moe_forward_static(const moe_config* cfg, const moe_weights* w, const uint16_t* x_bf16,
                              uint16_t* out_bf16, int32_t rows, void* stream);

/* The layer over any number of rows, in sub-chunks of the most rows one
 * moe_forward call takes for cfg (min(MOE_MAX_ROWS, MOE_MAX_IDS / top_k,
 * MOE_MAX_CHUNK_ROWS / ceil(hidden / 2048))) consecutive rows, each one
 * moe_forward on ``stream``
 * with ``ws``, in row order ("Function forward_moe" rustdoc, "WIDENED
 * (2026-08-31)" note: the 8-row batched prefill sub-chunk amortises its
 * routed experts over its own union).  x[rows, h] in, out[rows, h] out; rows
 * >= 1.  Arguments, refusals and ownership as moe_forward (x and out must not
 * overlap each other or the workspace).  Since every row's output depends on
 * that row alone, out is byte-identical to one-row calls.  The workspace holds
 * the last sub-chunk's intermediates. */
moe_status moe_forward_prefill(const moe_config* cfg, const moe_weights* w, const uint16_t* x_bf16,
                               uint16_t* out_bf16, int32_t rows, void* ws, size_t ws_bytes, void* stream);

/* The layer without the union: every (row, selected expert) pair is its own
 * slot, so an expert chosen by several rows is streamed once per row
 * (metrale_model_layers/layers/moe/forward_token_major.rs,
 * MoeLayer::forward_token_major_decode, evaluates the pairs this way).  It is
 * the baseline the union sweep is measured against ("Function forward_moe"
 * rustdoc, "RETRACTED (2026-08-29)" note: the same outputs either way).
 * Arguments, refusals and ownership as moe_forward; ``out`` is byte-identical
 * to moe_forward's.  The workspace's union fields hold the slot list instead
 * of the union: union_ids[t] = topk_ids[t], union_count = rows * top_k,
 * slot_to_union[t] = t, row_mask[t] = 1 << (t / top_k). */
moe_status moe_forward_token_major(const moe_config* cfg, const moe_weights* w, const uint16_t* x_bf16,
                                   uint16_t* out_bf16, int32_t rows, void* ws, size_t ws_bytes, void* stream);

/* One GPU's share of the layer under expert parallelism, before the
 * all-reduce (forward_token_major.rs under EP: the weighted sum is blended
 * with a zeroed shared term, then the output is all-reduced across ranks).
 * Every GPU routes all rows identically; this one sweeps only the union
 * experts in [expert_lo, expert_hi) and writes
 *   partial[r][n] = fp32( sum over j with expert_lo <= ids[r,j] < expert_hi
 *                         of w[r,j] * FFN_{ids[r,j]}(x_r)[n] )   (ascending j)
 *   partial  [rows, h] fp32 out, 16-byte aligned, overwritten.
 * It also runs the shared expert and leaves it, and the gate, in the
 * workspace for moe_ep_combine.  The expert tables are indexed by global
 * expert id; entries outside the range are read but never dereferenced.
 * Refusals as moe_forward, plus 0 <= expert_lo <= expert_hi <= num_experts.
 * The workspace's union fields hold the local union (moe_union_local). */
moe_status moe_forward_ep_partial(const moe_config* cfg, const moe_weights* w, const uint16_t* x_bf16,
                                  float* partial, int32_t rows, int32_t expert_lo, int32_t expert_hi, void* ws,
                                  size_t ws_bytes, void* stream);

/* After the caller's all-reduce of the ranks' partials (the reduce itself is
 * not part of this library): the shared expert added to the reduced routed
 * sum, as forward_token_major.rs does with moe_batched_blend (or residual_add,
 * gate 1, when shared_expert_gate is NULL):
 *   out[r][n] = bf16( reduced[r][n] + gate_r * FFN_shared(x_r)[n] )
 *   reduced  [rows, h] fp32 in, 16-byte aligned
 *   out      [rows, h] bf16 out, 16-byte aligned, overwritten
 * ``ws`` must hold what moe_forward_ep_partial left in it for the same x and
 * rows (same stream, no other call on the workspace in between). */
moe_status moe_ep_combine(const moe_config* cfg, const float* reduced, uint16_t* out_bf16, int32_t rows, void* ws,
                          size_t ws_bytes, void* stream);

/* moe_forward whose stage i kernel records ``stage_events[2i]`` (a
 * hipEvent_t, may be NULL) when it starts and ``stage_events[2i+1]`` when it
 * ends (hipExtLaunchKernel's start and stop events: the kernel's own
 * execution, with nothing enqueued between kernels).  2 * moe_num_stages()
 * entries.  ``stage_events`` itself may be NULL (then identical to
 * moe_forward). */
moe_status moe_forward_timed(const moe_config* cfg, const moe_weights* w, const uint16_t* x_bf16,
                             uint16_t* out_bf16, int32_t rows, void* ws, size_t ws_bytes,
                             void* stream, void* const* stage_events);

/* Measurement aid: the achievable streaming-read rate.  Reads every byte of
 * src[0, bytes) once with the sweeps' 16-byte non-temporal loads and writes
 * one fold word per block to sink[0, moe_read_probe_sink_words()).  Time it
 * with events on ``stream``; bytes / time is the read ceiling the layer's
 * weight sweeps are compared with.  src 16-byte aligned, bytes a positive
 * multiple of 16; sink must not overlap src. */
moe_status moe_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);
int32_t moe_read_probe_sink_words(void);

/* Number of kernel stages moe_forward enqueues, and the name of stage i
 * (NULL when out of range). */
int32_t moe_num_stages(void);
const char* moe_stage_name(int32_t i);

/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
