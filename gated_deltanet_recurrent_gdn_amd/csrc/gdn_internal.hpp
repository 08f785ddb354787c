// gdn_internal.hpp -- host-side launchers shared between the translation
// units of libgdn.so (not part of the public ABI; see include/gdn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "gdn.h"

namespace gdn {

// Launch with the error of THIS launch returned (not a stale runtime error).
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                  hipStream_t stream, Args&&... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<KArgs...> a(std::forward<Args>(args)...);
    void* p[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
    std::apply([&](auto&... e) { int i = 0; ((p[i++] = static_cast<void*>(&e)), ...); }, a);
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, p, shmem, stream);
}

// Source of the per-(token, value head) log-decay g and write strength beta:
// the arrays g, beta [rows, HV] fp32, or, when `a` is non-null, fused gating
// from the projections a, b [rows, HV] (bf16 when ab_bf16, else fp32) and the
// per-head A_log, dt_bias [HV] fp32.
struct GateArgs {
    const float* g;
    const float* beta;
    const void* a;
    const void* b;
    const float* A_log;
    const float* dt_bias;
    int32_t ab_bf16;
};

// Writes *err_flag (0 or GDN_EFLAG_* bits) for n slot indices and, when cu is
// non-null, cu_seqlens[n_cu + 1] against total.
hipError_t launch_validate(const int32_t* slot_idx, int32_t n, int32_t num_slots,
                           const int32_t* cu_seqlens, int32_t n_cu, int32_t total,
                           int32_t* err_flag, hipStream_t stream);

// Conv update, one token per row (decode).  out_dt may be GDN_F32 / GDN_BF16.
hipError_t launch_conv_decode(const void* x, gdn_dtype x_dt, const int32_t* slot_idx,
                              int32_t rows, void* conv_state, gdn_dtype cs_dt,
                              const void* weight, const void* bias, gdn_dtype w_dt,
                              void* out, gdn_dtype out_dt, int32_t dim, int32_t flags,
                              const int32_t* err_flag, hipStream_t stream);

// Conv update over token runs described by cu_seqlens.
hipError_t launch_conv_varlen(const void* x, gdn_dtype x_dt, const int32_t* cu_seqlens,
                              int32_t n_seqs, int32_t total_tokens, const int32_t* slot_idx,
                              void* conv_state, gdn_dtype cs_dt, const void* weight,
                              const void* bias, gdn_dtype w_dt, void* out, gdn_dtype out_dt,
                              int32_t dim, int32_t flags, const int32_t* err_flag,
                              hipStream_t stream);

// Gated delta-rule decode update from the post-conv activations y [B, D].
hipError_t launch_decode_rec(const void* y, gdn_dtype y_dt, const GateArgs& gate,
                             const int32_t* slot_idx, int32_t batch, float* rec_state,
                             void* out, gdn_dtype out_dt, const gdn_dims& dims, float scale,
                             int32_t flags, const int32_t* err_flag, hipStream_t stream);

// Fused decode step (conv + SiLU + norms + recurrence in one kernel, one
// workgroup per (row, key head) group, activations in LDS).  Chosen when
// dk <= 128, there is at least one group per 4 CUs and a group's activations
// fit in LDS; its results equal those of the conv + recurrence pair bitwise.
bool decode_step_fused_fits(const gdn_dims& d);
bool decode_step_use_fused(const gdn_dims& d, int32_t batch);
hipError_t launch_decode_step_fused(const void* x, gdn_dtype x_dt, const GateArgs& gate,
                                    const int32_t* slot_idx, int32_t batch,
                                    void* conv_state, gdn_dtype cs_dt, const void* weight,
                                    const void* bias, gdn_dtype w_dt, float* rec_state, void* out,
                                    gdn_dtype out_dt, const gdn_dims& dims, float scale,
                                    int32_t flags, const int32_t* err_flag, hipStream_t stream);

// Compute units of the current device (asked of the runtime each call).
int cu_count();

// Chunked prefill: one workgroup per (sequence, value head).
bool prefill_supported(const gdn_dims& d, gdn_dtype in_dt);
// q, k rows are sqk elements apart and v rows sv (H dk and HV dv for separate
// tensors; the conv width when they are slices of one activation row).
hipError_t launch_prefill(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                          const GateArgs& gate, const int32_t* cu, int32_t n_seqs,
                          const int32_t* slot, float* rec, void* out, gdn_dtype out_dt,
                          const gdn_dims& d, int32_t sqk, int32_t sv, float scale, int32_t flags,
                          const int32_t* err, hipStream_t st);

// Segment-parallel prefill.  Segment 0 of a sequence is its first `head`
// tokens, segments 1.. the following runs of seg_len tokens (head >= seg_len,
// both multiples of the 64-token chunk, so the chunks are those of the
// whole-sequence run; head == seg_len gives equal segments).  A segment maps
// its start state affinely, S_end = S_start P + B, with P the segment's run
// from the identity with v = 0 and B its run from the zero state.  Pass 1
// runs, in parallel, segment 0 from the slot's state (outputs written, end
// state kept) and every middle segment's P and B runs (no outputs); a scan
// composes the start states; pass 2 reruns segments 1.. from their start
// states with outputs, the last one writing the slot.  The workspace holds
// three D x D fp32 matrices (start state, P, B) per (segment id, value head);
// the segment id of segment j of sequence n is n + cu[n] / seg_len + j, below
// n_seqs + total / seg_len + 1.
struct PrefillSchedule {
    int32_t seg_len;     // 0: whole sequences
    int32_t head;        // tokens of segment 0 (>= seg_len)
    bool paired;         // pass 1: a middle segment's P and B runs in one workgroup
};
int64_t prefill_segment_ids(int32_t n_seqs, int32_t total_tokens, int32_t seg_len);
size_t prefill_segmented_workspace(const gdn_dims& d, int32_t n_seqs, int32_t total_tokens,
                                   int32_t seg_len);
// Whether the two segment passes' grids (bounded from the sizes alone) stay
// within the 65535 workgroups of a grid's y extent.
bool prefill_seg_grid_fits(int32_t n_seqs, int32_t total_tokens, PrefillSchedule sch);
// Schedule the plain prefill call uses for these sizes (seg_len 0: whole
// sequences), from a model of its workgroup rounds on the current device.
PrefillSchedule prefill_auto_schedule(const gdn_dims& d, int32_t n_seqs, int32_t total_tokens);
hipError_t launch_prefill_segmented(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                                    const GateArgs& gate, const int32_t* cu, int32_t n_seqs,
                                    int32_t total_tokens, const int32_t* slot, float* rec,
                                    void* out, gdn_dtype out_dt, const gdn_dims& d,
                                    int32_t sqk, int32_t sv, float scale, int32_t flags,
                                    PrefillSchedule sch, float* ws, const int32_t* err,
                                    hipStream_t st);

// Gated RMSNorm over rows of `dim` values (z has x's dtype; NULL = no gate).
hipError_t launch_gated_rmsnorm(const void* x, gdn_dtype x_dt, const void* z, const void* w,
                                gdn_dtype w_dt, void* out, gdn_dtype out_dt, int64_t rows,
                                int32_t dim, float eps, int32_t flags, hipStream_t st);

}  // namespace gdn
