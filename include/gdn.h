/*
 * gdn.h -- C ABI of libgdn.so, the MI355X (gfx950) Gated DeltaNet core.
 *
 * Operations, each a thin host layer over hand-written HIP kernels:
 *   gdn_conv_update      causal depthwise conv1d over a slot-indexed conv cache
 *   gdn_decode_step      one decode token per row: conv -> SiLU -> q/k L2 norm
 *                        -> gated delta-rule update of a slot-indexed fp32 state
 *   gdn_decode_recurrent the recurrent half of the decode step alone
 *   gdn_prefill_chunked  varlen chunked (64-token, WY/UT) prefill on post-conv
 *                        q/k/v, reading and writing the same state cache
 *   gdn_decode_step_gated, gdn_prefill_chunked_gated
 *                        the same two calls with the gating fused in: g and
 *                        beta computed in-kernel from the raw projections
 *   gdn_mixed_step       one step holding decode rows and prefill sequences,
 *                        the decode rows computed exactly as in a decode-only
 *                        step
 *   gdn_prefill_segmented
 *                        the chunked prefill on an explicit segment-parallel
 *                        schedule (the plain call picks one by itself)
 *   gdn_gated_rmsnorm    the gated RMSNorm epilogue after the core
 *   gdn_decode_step_noalloc
 *                        gdn_decode_step for callers that cannot allocate
 *
 * Sources (pages, by title and section):
 *   [P1] RL-Kernel PR #469 "C6: GDN decode-step goldens and recurrent/conv
 *        state contract": "Summary" (gating, GQA map, QK norm, state layouts),
 *        "State ABI: index validation and the two NULL_BLOCK_ID contracts",
 *        "The conv half: coverage and the two mismatch mechanisms".
 *   [P2] "A reduction barrier makes Qwen GDN graph replay bit exact" (replay
 *        determinism; inactive rows and slot 0 left untouched).
 *   [P4] vLLM PR #53864, "Numerical root cause and fix" (16x16 lower-
 *        triangular KK^T diagonal-block inverses in the chunked prefill).
 *   The recurrence is the gated delta rule
 *        S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *        o_t = S_t q_t,
 *   computed as S1 = exp(g) S, u = S1 k, S' = S1 + beta (v - u) k^T, o = S' q.
 *
 * Conventions common to every call
 *   - Every tensor is caller-owned DEVICE memory, dense, row-major (C order),
 *     at least 16-byte aligned.  The library never allocates, frees or
 *     synchronises and holds no state between calls (the one exception is
 *     gdn_decode_step_noalloc's per-device scratch array, declared with that
 *     call for callers that cannot allocate); each call only enqueues
 *     kernels (and, in gdn_mixed_step, event records and waits) on the
 *     caller's `stream` (NULL = the default stream) and streams, and returns.
 *     Calls on different streams that touch disjoint slots and buffers are
 *     independent.
 *   - Caches are updated in place.  Outputs must not alias any input.  Within
 *     one call each active slot may appear at most once ([P1] "State ABI").
 *   - Slot indices: s <= 0 marks an inactive (padded) row: its outputs are
 *     written as zeros and no cache entry is read or written.  Slot 0 is the
 *     reserved null block and is never addressed ([P1] "State ABI"; [P2]).
 *   - Synchronous status (gdn_status): what the host can check without reading
 *     device memory -- null pointers, dims, dtypes, alignment, workspace size.
 *     Those argument errors are found before anything is enqueued.
 *     GDN_ERR_LAUNCH (the runtime refused a launch) can leave the kernels the
 *     call launched before that one enqueued.
 *   - Device-side validation: with GDN_FLAG_VALIDATE set, a first kernel
 *     checks the slot indices (and cu_seqlens) and WRITES *err_flag (0 when
 *     clean, else GDN_EFLAG_* bits).  When any bit is set every later kernel
 *     of the call returns before touching outputs or caches (fail closed).
 *     err_flag is then a required int32 device pointer; read it after the
 *     stream completes.  Without the flag, indices are trusted (as the
 *     serving providers of [P1] do) and err_flag may be NULL.
 *   - Results are bitwise reproducible run to run and batch-invariant: a row's
 *     outputs and cache updates do not depend on which other rows share the
 *     call, their order, or the batch size (fixed per-row reduction order, no
 *     split reductions, no atomics on data).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

/* HIP stream and event handles: the runtime's own opaque pointer types (the
   same declarations as hip_runtime_api.h, repeated only when that header is
   not already in scope). */
#ifndef HIP_INCLUDE_HIP_HIP_RUNTIME_API_H
typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,       /* a required pointer is NULL                        */
    GDN_ERR_DIMS = 2,       /* unsupported or inconsistent sizes                 */
    GDN_ERR_DTYPE = 3,      /* unsupported dtype (combination)                   */
    GDN_ERR_ALIGN = 4,      /* a pointer is not 16-byte aligned                  */
    GDN_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than *_workspace_size   */
    GDN_ERR_LAUNCH = 6,     /* the HIP runtime refused a kernel launch           */
    GDN_ERR_FLAGS = 7       /* unknown flag bits, or VALIDATE without err_flag   */
} gdn_status;

enum {
    GDN_FLAG_SILU = 1,      /* SiLU after the conv (decode step, conv update)    */
    GDN_FLAG_QK_L2NORM = 2, /* q, k <- x / sqrt(sum(x*x) + 1e-6) before use      */
    GDN_FLAG_VALIDATE = 4,  /* device-side index validation, see above           */
    GDN_FLAG_STEP_FUSED = 8,  /* gdn_decode_step: force the one-kernel path      */
    GDN_FLAG_STEP_SPLIT = 16, /* gdn_decode_step: force conv kernel + recurrence  */
    GDN_FLAG_PREFILL_NS3 = 32, /* prefill A/B variant: diagonal KK^T blocks by   */
    GDN_FLAG_PREFILL_NS4 = 64, /* 3 or 4 bf16 Newton-Schulz rounds (see below)   */
    GDN_FLAG_PREFILL_SEQUENTIAL = 128, /* prefill: never split sequences into     */
                                       /* segments (see gdn_prefill_chunked)      */
    GDN_FLAG_PREFILL_SINGLE_ROLE = 256 /* prefill: run the chunk step on the      */
                                       /* single-role kernel (see below)          */
};

enum {                      /* flags of gdn_gated_rmsnorm                         */
    GDN_NORM_GATE_SIGMOID = 1,  /* gate = sigmoid(z) instead of SiLU(z)           */
    GDN_NORM_ZERO_CENTRED = 2   /* weight enters as weight + 1                    */
};

enum {                      /* bits written to *err_flag under GDN_FLAG_VALIDATE */
    GDN_EFLAG_SLOT_RANGE = 1,   /* an active slot >= num_slots                   */
    GDN_EFLAG_SLOT_REPEAT = 2,  /* an active slot appears twice                  */
    GDN_EFLAG_SEQLENS = 4       /* cu_seqlens[0] != 0, decreasing, or last != total */
};

/* Head geometry.  conv channel count D = 2*num_k_heads*head_k_dim +
   num_v_heads*head_v_dim, channel order [q | k | v], each head-major with the
   head dimension contiguous.  Value head hv reads key head hv / (HV / H)
   ([P1] "How the golden relates to the kernel": no repeat_interleave).
   Supported: head_k_dim in {32, 64, 128, 256}; head_v_dim a multiple of 32,
   at most 256; HV a multiple of H; conv_width == 4. */
typedef struct {
    int32_t num_k_heads;   /* H  */
    int32_t num_v_heads;   /* HV */
    int32_t head_k_dim;    /* dk */
    int32_t head_v_dim;    /* dv */
    int32_t conv_width;    /* W  */
} gdn_dims;

/* Inputs of the fused gating ([P1] "How the golden relates to the kernel",
   item 1), computed in fp32 inside the kernels for each (row or token r,
   value head h):
     beta[r, h] = 1 / (1 + exp(-b[r, h]))
     g[r, h]    = -exp(A_log[h]) * softplus(a[r, h] + dt_bias[h]),
     softplus(x) = x for x > 20, else log(1 + exp(x)) (evaluated as log1p).
   All device memory, caller-owned, read only.  a and b have the layout of the
   g and beta arrays they replace ([rows, HV]); no alignment beyond the
   element's own is needed. */
typedef struct {
    const void* a;           /* [rows, HV] ab_dt: decay-gate pre-activation  */
    const void* b;           /* [rows, HV] ab_dt: beta pre-activation        */
    gdn_dtype ab_dt;         /* GDN_F32 or GDN_BF16                          */
    const float* A_log;      /* [HV] fp32                                    */
    const float* dt_bias;    /* [HV] fp32                                    */
} gdn_gate_inputs;

/*
 * gdn_conv_update -- causal depthwise conv1d with per-slot left context
 * ([P1] "Summary": conv state [num_blocks, dim, W-1]; "The conv half").
 *
 *   x           [total_tokens, dim], x_dt
 *   cu_seqlens  [n_seqs + 1] int32 token offsets, or NULL: one token per row
 *               (n_seqs == total_tokens, decode)
 *   slot_idx    [n_seqs] int32 (<= 0 inactive)
 *   conv_state  [num_slots, dim, width-1], cs_dt, oldest tap first.  Rolled in
 *               place to the last width-1 raw inputs of each active sequence
 *               (an exact copy in cs_dt: bit-exact roll); a zero-length active
 *               sequence leaves its state unchanged.
 *   weight      [dim, width], bias [dim] or NULL, both w_dt.  Tap j multiplies
 *               X[t + j] where X = [conv_state row, tokens]: tap width-1 is the
 *               current token.
 *   out         [total_tokens, dim], out_dt:
 *               y = bias + sum_j weight[c, j] X[t + j] accumulated in fp32 in
 *               tap order j = 0..W-1 starting from the bias, then SiLU when
 *               GDN_FLAG_SILU; rows of inactive sequences are zeros.
 *   dtypes      x, conv_state, weight: GDN_F32 or GDN_BF16 each; out likewise.
 *   flags       GDN_FLAG_SILU | GDN_FLAG_VALIDATE.
 */
gdn_status gdn_conv_update(const void* x, gdn_dtype x_dt,
                           const int32_t* cu_seqlens, int32_t n_seqs, int32_t total_tokens,
                           const int32_t* slot_idx,
                           void* conv_state, gdn_dtype cs_dt, int32_t num_slots,
                           const void* weight, const void* bias, gdn_dtype w_dt,
                           void* out, gdn_dtype out_dt,
                           int32_t dim, int32_t width, int32_t flags,
                           int32_t* err_flag, hipStream_t stream);

/*
 * gdn_decode_workspace_size -- bytes of device workspace gdn_decode_step needs
 * for `batch` rows (the fp32 post-conv activations, batch * D * 4 bytes,
 * rounded up to 256).  Returns 0 for unsupported dims.
 */
size_t gdn_decode_workspace_size(const gdn_dims* dims, int32_t batch);

/*
 * gdn_decode_step -- one decode token per row ([P1] "Summary"; the decode-only
 * step: conv update, SiLU, split, QK norm with scale on q, recurrent update).
 *
 *   mixed_qkv    [batch, D], x_dt (GDN_F32 or GDN_BF16)
 *   g, beta      [batch, HV] fp32: alpha = exp(g) decays the state, beta is
 *                the write strength (already gated by the caller)
 *   slot_idx     [batch] int32 (<= 0 inactive: zero output, caches untouched)
 *   conv_state   [num_slots, D, W-1] cs_dt; conv_weight [D, W], conv_bias [D]
 *                or NULL, w_dt
 *   rec_state    [num_slots, HV, dv, dk] fp32 (S[v][k], k fastest), in place
 *   out          [batch, HV, dv], out_dt (GDN_F32 or GDN_BF16)
 *   scale        multiplies q after the norm (k is never scaled); usually
 *                dk^-1/2
 *   flags        GDN_FLAG_SILU | GDN_FLAG_QK_L2NORM | GDN_FLAG_VALIDATE, and
 *                at most one of GDN_FLAG_STEP_FUSED / GDN_FLAG_STEP_SPLIT
 *   workspace    >= gdn_decode_workspace_size(dims, batch) bytes of device
 *                memory, contents irrelevant; not retained after the call
 *
 * Two kernel paths compute the step, with bitwise-identical results: a fused
 * kernel (one workgroup per (row, key head) group: conv of q_h, k_h and the
 * value heads sharing h into LDS, then their recurrence) and a conv kernel
 * writing the fp32 activations to the workspace followed by the recurrence
 * kernel.  By default the fused kernel runs when head_k_dim <= 128, when
 * batch * num_k_heads is between a quarter of the number of compute units
 * and that number (one or two groups per compute unit at most: there its
 * double-buffered passes hide its latency chain; with more groups the pair's
 * small recurrence items stream the state faster) and when
 * (2 dk + (HV / H) (dv + 2)) * 4 bytes fit in 64 KiB of LDS
 * (gdn_decode_step_fused reports the choice); the STEP flags
 * force a path (GDN_ERR_DIMS if the fused kernel is forced where the group
 * does not fit, GDN_ERR_FLAGS if both are set).
 */
gdn_status gdn_decode_step(const void* mixed_qkv, gdn_dtype x_dt,
                           const float* g, const float* beta,
                           const int32_t* slot_idx, int32_t batch,
                           void* conv_state, gdn_dtype cs_dt,
                           const void* conv_weight, const void* conv_bias, gdn_dtype w_dt,
                           float* rec_state, int32_t num_slots,
                           void* out, gdn_dtype out_dt,
                           const gdn_dims* dims, float scale, int32_t flags,
                           void* workspace, size_t workspace_bytes,
                           int32_t* err_flag, hipStream_t stream);

/*
 * gdn_decode_step_fused -- the path gdn_decode_step, gdn_decode_step_gated and
 * the decode rows of gdn_mixed_step take for `batch` rows without a STEP flag
 * on the current device: 1 = the fused kernel, 0 = the conv kernel followed by
 * the recurrence kernel (the rule above: dims, batch and the device's compute
 * unit count alone; both paths give the same bits).  -1 for invalid dims or a
 * batch outside [0, 65535].  Enqueues nothing.
 */
int32_t gdn_decode_step_fused(const gdn_dims* dims, int32_t batch);

/*
 * gdn_decode_step_noalloc -- gdn_decode_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and bitwise the same results.  Where the call takes the conv +
 * recurrence pair, the fp32 activations (batch * D * 4 bytes) go to a scratch
 * array of GDN_NOALLOC_SCRATCH_BYTES that the library holds in device memory,
 * one per device, until the process ends.  Where they would not fit (at
 * D = 8192: more than 512 rows) the call takes the fused kernel instead,
 * which needs no scratch and gives the same bits; GDN_ERR_WORKSPACE if
 * GDN_FLAG_STEP_SPLIT forces the pair there (or the fused kernel's group does
 * not fit its LDS).  The call allocates nothing; its first call on a device looks
 * up the array's device address (GDN_ERR_LAUNCH if the runtime cannot) and
 * keeps it for that device.  Every call on a device shares that device's
 * array, so calls that can overlap on one device (different streams, or
 * threads) race on it: order them, or use gdn_decode_step.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (16u << 20)
gdn_status gdn_decode_step_noalloc(const void* mixed_qkv, gdn_dtype x_dt,
                                   const float* g, const float* beta,
                                   const int32_t* slot_idx, int32_t batch,
                                   void* conv_state, gdn_dtype cs_dt,
                                   const void* conv_weight, const void* conv_bias, gdn_dtype w_dt,
                                   float* rec_state, int32_t num_slots,
                                   void* out, gdn_dtype out_dt,
                                   const gdn_dims* dims, float scale, int32_t flags,
                                   int32_t* err_flag, hipStream_t stream);

/*
 * gdn_decode_recurrent -- the recurrent half of the decode step alone, on
 * post-conv activations (the split of [P1] "Which provider this aligns to":
 * conv update, then the packed recurrent decode on mixed q|k|v):
 * split [q | k | v] -> QK norm (flag) -> scale q -> gated delta rule on
 * rec_state[slot] -> o.  gdn_decode_step == gdn_conv_update (one token per
 * row, SiLU, fp32 output) followed by this call, bit for bit.
 *
 *   qkv          [batch, D], qkv_dt (GDN_F32 or GDN_BF16)
 *   g, beta      [batch, HV] fp32; slot_idx [batch] int32 (<= 0 inactive)
 *   rec_state    [num_slots, HV, dv, dk] fp32, in place
 *   out          [batch, HV, dv], out_dt
 *   flags        GDN_FLAG_QK_L2NORM | GDN_FLAG_VALIDATE
 */
gdn_status gdn_decode_recurrent(const void* qkv, gdn_dtype qkv_dt,
                                const float* g, const float* beta,
                                const int32_t* slot_idx, int32_t batch,
                                float* rec_state, int32_t num_slots,
                                void* out, gdn_dtype out_dt,
                                const gdn_dims* dims, float scale, int32_t flags,
                                int32_t* err_flag, hipStream_t stream);

/*
 * gdn_prefill_workspace_size -- bytes of device workspace with which
 * gdn_prefill_chunked(_gated) runs the segment-parallel schedule (see
 * gdn_prefill_segmented) for n_seqs sequences and total_tokens tokens on the
 * current device; 0 when those sizes run whole sequences (the sequences are
 * short) and for unsupported dims.  The schedule depends on the sizes only:
 *   - few (sequence, value head) runs (n_seqs * HV at most half the compute
 *     units): equal segments, where a model of the workgroup rounds gains;
 *   - a busy chip: segment 0 of each sequence is a head of the chunks a
 *     compute unit carries when the work is spread evenly, and the tokens past
 *     it form segments of about a quarter of that; sequences no longer than
 *     the head run whole, so equal lengths keep whole runs, while the tails of
 *     longer ones run in parallel on the units shorter ones free.
 */
size_t gdn_prefill_workspace_size(const gdn_dims* dims, int32_t n_seqs, int32_t total_tokens);

/*
 * gdn_prefill_chunked -- varlen chunked prefill on post-conv q, k, v.
 * Equal (to rounding) to running the decode recurrence token by token; the
 * sequence is cut into 64-token chunks, each handled in WY/UT form with
 * inverses of the 16x16 lower-triangular KK^T diagonal blocks by exact fp32
 * forward substitution ([P4] "Numerical root cause and fix"), and the state is
 * carried from chunk to chunk.
 *
 *   q, k         [total_tokens, H, dk]; v [total_tokens, HV, dv]; in_dt:
 *                GDN_BF16 at dk = dv in {32, 64, 128}; GDN_F32 only at 32 and
 *                64 (GDN_ERR_DTYPE at 128).  fp32 inputs are carried as bf16
 *                hi + lo planes in LDS, and at 128 the doubled K, Q, K^T and
 *                V^T planes alone (8 x 64 x 128 x 2 bytes = 128 KiB) leave too
 *                little of the 160 KiB of LDS for the chunk's work arrays;
 *                round fp32 inputs to bf16 first at that size.
 *   g, beta      [total_tokens, HV] fp32
 *   cu_seqlens   [n_seqs + 1] int32; slot_idx [n_seqs] int32 (<= 0 inactive:
 *                zero outputs, state untouched)
 *   rec_state    [num_slots, HV, dv, dk] fp32: each active sequence starts
 *                from rec_state[slot] and its final state is written back
 *                there (zero-fill a fresh slot first)
 *   out          [total_tokens, HV, dv], out_dt
 *   scale, flags as for gdn_decode_step (GDN_FLAG_QK_L2NORM, GDN_FLAG_VALIDATE),
 *                plus at most one of GDN_FLAG_PREFILL_NS3 / GDN_FLAG_PREFILL_NS4: a
 *                numerics A/B variant that inverts the 16x16 diagonal KK^T blocks
 *                by 3 or 4 Newton-Schulz rounds with bf16 intermediates, as [P4]
 *                "Numerical root cause and fix" describes, instead of the default
 *                exact fp32 forward substitution
 *                or GDN_FLAG_PREFILL_SEQUENTIAL, and GDN_FLAG_PREFILL_SINGLE_ROLE:
 *                at dk = dv = 128 with bf16 inputs the chunk step normally runs
 *                on a kernel whose waves split into two roles (half carry the
 *                state and produce outputs, half build the next chunk's
 *                coefficients ahead of them); this flag runs it on the
 *                single-role kernel instead, which computes the same values
 *                bit for bit (an A/B switch for tests and timing)
 *   workspace    device memory, 16-byte aligned, or NULL.  With at least
 *                gdn_prefill_workspace_size(...) bytes (and that size > 0,
 *                and no GDN_FLAG_PREFILL_SEQUENTIAL) the call runs the
 *                segment-parallel schedule of gdn_prefill_segmented with the
 *                head and segment lengths the library picks for these sizes
 *                (from n_seqs, total_tokens, the head dims and the device's CU
 *                count alone); otherwise
 *                each (sequence, value head) is walked by one workgroup from
 *                start to end.  The two schedules agree to rounding, not
 *                bitwise: whole-sequence runs are bitwise independent of how a
 *                sequence is split into calls along the 64-token grid.
 */
gdn_status gdn_prefill_chunked(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                               const float* g, const float* beta,
                               const int32_t* cu_seqlens, int32_t n_seqs, int32_t total_tokens,
                               const int32_t* slot_idx,
                               float* rec_state, int32_t num_slots,
                               void* out, gdn_dtype out_dt,
                               const gdn_dims* dims, float scale, int32_t flags,
                               void* workspace, size_t workspace_bytes,
                               int32_t* err_flag, hipStream_t stream);

/*
 * gdn_prefill_segmented -- gdn_prefill_chunked with the sequences cut into
 * segments that are processed in parallel: segment 0 is the first head_len
 * tokens of the sequence and segments 1.. the following runs of seg_len
 * tokens (both multiples of 64, so the segments are runs of whole 64-token
 * chunks; head_len 0 means seg_len; a sequence of at most head_len tokens is
 * one segment and runs whole).  A segment
 * maps its start state affinely: S_end = S_start P + B, where P is the
 * segment's run from the identity with v = 0 and B its run from the zero state
 * (the token update multiplies the state on the right by
 * exp(g)(I - beta k k^T) and adds beta v k^T; [P1] "Notes" and "Deliberately
 * not in this PR" mention a context-parallel prefill path without describing
 * it; this is a one-GPU form of such a split).  Three launches:
 * segment 0 from the slot's state together with the P and B runs of the
 * middle segments; a scan of the start states in fp32; segments 1.. again
 * from their start states, writing outputs and, for the last, the slot.
 * A middle segment costs its P run, its B run and its rerun (at dk = 128 the
 * P and B runs are workgroups of their own; at 32 and 64 they share one), for
 * a critical path of about the head plus one segment instead of the whole
 * sequence.
 *
 *   g, beta, gate  either g and beta (gate NULL) or gate (g, beta NULL; as in
 *                  gdn_prefill_chunked_gated); GDN_ERR_FLAGS if both
 *   seg_len        tokens per segment: GDN_ERR_DIMS unless a positive multiple
 *                  of 64, at most 32768 segments of total_tokens, and the first
 *                  pass's workgroup rows, n_seqs + (2 at dk = 128, else 1) x
 *                  (total_tokens / seg_len + n_seqs), at most 65535
 *   head_len       tokens of segment 0: 0 (= seg_len) or a multiple of 64 of
 *                  at least seg_len (GDN_ERR_DIMS otherwise)
 *   workspace      >= gdn_prefill_segmented_workspace_size(dims, n_seqs,
 *                  total_tokens, seg_len) bytes of device memory, 16-byte
 *                  aligned: three dv x dk fp32 matrices per (segment id, value
 *                  head), (n_seqs + total_tokens / seg_len + 1) segment ids
 *                  (GDN_ERR_WORKSPACE if NULL or smaller, with tokens to run)
 * Every other argument, flag (GDN_FLAG_PREFILL_SEQUENTIAL excepted:
 * GDN_ERR_FLAGS) and error is as for gdn_prefill_chunked.
 */
size_t gdn_prefill_segmented_workspace_size(const gdn_dims* dims, int32_t n_seqs,
                                            int32_t total_tokens, int32_t seg_len);
gdn_status gdn_prefill_segmented(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                                 const float* g, const float* beta, const gdn_gate_inputs* gate,
                                 const int32_t* cu_seqlens, int32_t n_seqs, int32_t total_tokens,
                                 const int32_t* slot_idx,
                                 float* rec_state, int32_t num_slots,
                                 void* out, gdn_dtype out_dt,
                                 const gdn_dims* dims, float scale, int32_t flags,
                                 int32_t seg_len, int32_t head_len,
                                 void* workspace, size_t workspace_bytes,
                                 int32_t* err_flag, hipStream_t stream);

/*
 * gdn_decode_step_gated / gdn_prefill_chunked_gated -- gdn_decode_step and
 * gdn_prefill_chunked with the gating fused in ([P1] "How the golden relates
 * to the kernel", item 1): `gate` (host pointer to a gdn_gate_inputs whose
 * arrays are device memory) replaces the g and beta arrays; every other
 * argument, the error codes and the fail-closed behaviour are as in the
 * ungated call.  GDN_ERR_NULL if gate is NULL or, with rows to process, any
 * of its arrays is; GDN_ERR_DTYPE if ab_dt is not GDN_F32 / GDN_BF16.
 */
gdn_status gdn_decode_step_gated(const void* mixed_qkv, gdn_dtype x_dt,
                                 const gdn_gate_inputs* gate,
                                 const int32_t* slot_idx, int32_t batch,
                                 void* conv_state, gdn_dtype cs_dt,
                                 const void* conv_weight, const void* conv_bias, gdn_dtype w_dt,
                                 float* rec_state, int32_t num_slots,
                                 void* out, gdn_dtype out_dt,
                                 const gdn_dims* dims, float scale, int32_t flags,
                                 void* workspace, size_t workspace_bytes,
                                 int32_t* err_flag, hipStream_t stream);

gdn_status gdn_prefill_chunked_gated(const void* q, const void* k, const void* v,
                                     gdn_dtype in_dt, const gdn_gate_inputs* gate,
                                     const int32_t* cu_seqlens, int32_t n_seqs,
                                     int32_t total_tokens, const int32_t* slot_idx,
                                     float* rec_state, int32_t num_slots,
                                     void* out, gdn_dtype out_dt,
                                     const gdn_dims* dims, float scale, int32_t flags,
                                     void* workspace, size_t workspace_bytes,
                                     int32_t* err_flag, hipStream_t stream);

/*
 * gdn_mixed_workspace_size -- bytes of device workspace gdn_mixed_step needs:
 * the decode rows' fp32 activations (n_dec * D * 4) and the prefill tokens'
 * bf16 activations (total_pre * D * 2), each rounded up to 256.  0 for
 * unsupported dims or negative sizes.
 */
size_t gdn_mixed_workspace_size(const gdn_dims* dims, int32_t n_dec, int32_t total_pre);

/*
 * gdn_mixed_step -- one serving step that holds both cached decode rows and
 * prefill sequences ([P1] "Not reproducible from this branch: the mixed
 * decode+prefill measurement": with the decode rows of a mixed step routed
 * through a different recurrent kernel, their state depended on the step's
 * composition; the proposed fix routes them through the decode kernel and
 * aligns non-final chunked-prefill calls to the 64-token grid).
 *
 * The decode rows run gdn_decode_step's kernels for n_dec rows (beside a
 * prefill part on prefill_stream, the fused kernel where it fits, which lets
 * the prefill's workgroups take compute units as the decode's groups retire;
 * both of that call's paths give the same bits), so every decode row's output,
 * recurrent state and conv state are bitwise independent of what else the
 * step holds and of the streams.  The prefill tokens go through
 * the varlen conv (SiLU per flags) into bf16 activations -- the serving path's
 * convention -- and then the chunked prefill: as one run per (sequence, value
 * head), or, when the step has no decode rows and the workspace also holds
 * the segment states, on the segment-parallel schedule that
 * gdn_prefill_chunked would pick (see gdn_prefill_workspace_size).  The
 * schedule depends on these arguments only, never on the streams.
 * With one run per sequence (the minimal workspace, decode rows in the step,
 * or GDN_FLAG_PREFILL_SEQUENTIAL) a sequence prefilled over several calls
 * equals one whole prefill bitwise when every non-final call covers a
 * multiple of 64 of its tokens (the chunk grid then coincides).
 *
 * Streams.  With prefill_stream NULL both parts run in order on `stream`
 * (fork_event and join_event are ignored).  With a prefill_stream and a step
 * holding both parts, the call records fork_event on `stream` after the
 * optional validation, makes prefill_stream wait for it, enqueues the prefill
 * part there and the decode part on `stream`, records join_event on
 * prefill_stream and makes `stream` wait for it: the parts overlap on the GPU
 * (they share no memory, active slots being distinct across both), and the
 * call is still ordered on `stream` as a whole, under stream capture too (the
 * fork pulls prefill_stream into the capture and the join ends it there).
 * Results are bitwise the same with or without a prefill_stream.  The streams
 * and events belong to the caller (events created with
 * hipEventDisableTiming are enough); one event pair must not be recorded by
 * two calls concurrently from different host threads.
 *
 *
 *   x            [n_dec + total_pre, D], x_dt: the n_dec decode rows, then the
 *                prefill tokens (pre-conv mixed q | k | v)
 *   g, beta      [n_dec + total_pre, HV] fp32, in the same row order
 *   n_dec        decode rows (one token each)
 *   cu_seqlens   [n_pre + 1] offsets of the prefill sequences within the
 *                total_pre prefill tokens (cu_seqlens[0] == 0); may be NULL
 *                when n_pre == 0
 *   slot_idx     [n_dec + n_pre]: the decode rows' slots, then the prefill
 *                sequences'; <= 0 inactive; active slots distinct across
 *                both parts
 *   conv_state, conv_weight, conv_bias, rec_state, num_slots, scale:
 *                as for gdn_decode_step (the prefill part reads and rolls
 *                the same conv cache and recurrent cache)
 *   out          [n_dec + total_pre, HV, dv], out_dt
 *   flags        GDN_FLAG_SILU | GDN_FLAG_QK_L2NORM | GDN_FLAG_VALIDATE (one
 *                validation over all slot indices and cu_seqlens), the
 *                decode rows' GDN_FLAG_STEP_FUSED / GDN_FLAG_STEP_SPLIT, and
 *                GDN_FLAG_PREFILL_SEQUENTIAL (one run per sequence always)
 *                and GDN_FLAG_PREFILL_SINGLE_ROLE (as for gdn_prefill_chunked)
 *   workspace    >= gdn_mixed_workspace_size(dims, n_dec, total_pre) bytes;
 *                with gdn_mixed_workspace_size(dims, n_dec, total_pre) +
 *                gdn_prefill_workspace_size(dims, n_pre, total_pre) bytes the
 *                prefill part may take the segment-parallel schedule (its
 *                segment states live past the activations)
 *   stream       the step's stream: validation, decode part and, without a
 *                prefill_stream, the prefill part
 *   prefill_stream, fork_event, join_event
 *                the caller's second stream and two events for the
 *                overlapped schedule above, or NULL, NULL, NULL
 *                (GDN_ERR_NULL if prefill_stream is given without both events)
 * The prefill part needs dk == dv <= 128 (GDN_ERR_DIMS otherwise, when
 * n_pre > 0).
 */
gdn_status gdn_mixed_step(const void* x, gdn_dtype x_dt,
                          const float* g, const float* beta,
                          int32_t n_dec,
                          const int32_t* cu_seqlens, int32_t n_pre, int32_t total_pre,
                          const int32_t* slot_idx,
                          void* conv_state, gdn_dtype cs_dt,
                          const void* conv_weight, const void* conv_bias, gdn_dtype w_dt,
                          float* rec_state, int32_t num_slots,
                          void* out, gdn_dtype out_dt,
                          const gdn_dims* dims, float scale, int32_t flags,
                          void* workspace, size_t workspace_bytes,
                          int32_t* err_flag, hipStream_t stream,
                          hipStream_t prefill_stream, hipEvent_t fork_event,
                          hipEvent_t join_event);

/*
 * gdn_gated_rmsnorm -- the gated RMSNorm that follows the GDN core in the
 * block ([P1] "Latest Status": zero-centred and gated RMSNorm with SiLU or
 * sigmoid gating; the pages print no formula, the plain definition is used,
 * the norm before the gate):
 *   out[r, j] = x[r, j] / sqrt(sum_j x[r, j]^2 / dim + eps) * w'[j] * act(z[r, j])
 *   w' = weight + 1 under GDN_NORM_ZERO_CENTRED, else weight;
 *   act = SiLU, or sigmoid under GDN_NORM_GATE_SIGMOID; z == NULL: no gate.
 *
 *   x            [rows, dim] x_dt (e.g. o viewed as [tokens * HV, dv])
 *   z            [rows, dim] in x_dt, or NULL
 *   weight       [dim] w_dt
 *   out          [rows, dim] out_dt; may be x itself (each row is read into
 *                registers before it is written)
 *   dim          a multiple of 4, 4 ... 1024; eps >= 0
 * Per-row fp32 arithmetic with a fixed reduction order: batch-invariant.
 */
gdn_status gdn_gated_rmsnorm(const void* x, gdn_dtype x_dt, const void* z,
                             const void* weight, gdn_dtype w_dt,
                             int64_t rows, int32_t dim, float eps, int32_t flags,
                             void* out, gdn_dtype out_dt, hipStream_t stream);

/* gdn_strerror -- static, NUL-terminated description of a status code. */
const char* gdn_strerror(gdn_status s);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
