// api.hip -- the extern "C" entry points of libgdn.so (declared in gdn.h).
//
// Host-side only: validate what can be checked without reading device memory,
// then enqueue the kernels on the caller's stream(s) and return.  No
// allocation, no synchronisation, no global mutable state: every stream and
// event a call uses is the caller's.
#include <hip/hip_runtime.h>

#include <atomic>

#include "gdn.h"
#include "gdn_internal.hpp"

using namespace gdn;

// gdn_decode_step_noalloc's scratch (see noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int32_t KNOWN_FLAGS = GDN_FLAG_SILU | GDN_FLAG_QK_L2NORM | GDN_FLAG_VALIDATE;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(gdn_dtype t) { return t == GDN_F32 || t == GDN_BF16; }
size_t round256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

gdn_status check_dims(const gdn_dims* d) {
    if (!d) return GDN_ERR_NULL;
    const int32_t H = d->num_k_heads, HV = d->num_v_heads, dk = d->head_k_dim, dv = d->head_v_dim;
    if (H <= 0 || HV <= 0 || HV % H != 0) return GDN_ERR_DIMS;
    if (dk != 32 && dk != 64 && dk != 128 && dk != 256) return GDN_ERR_DIMS;
    if (dv <= 0 || dv % 32 != 0 || dv > 256) return GDN_ERR_DIMS;
    if (d->conv_width != 4) return GDN_ERR_DIMS;
    const int64_t D = 2LL * H * dk + static_cast<int64_t>(HV) * dv;
    if (D > (1 << 20)) return GDN_ERR_DIMS;
    return GDN_OK;
}

int64_t conv_channels(const gdn_dims* d) {
    return 2LL * d->num_k_heads * d->head_k_dim + static_cast<int64_t>(d->num_v_heads) * d->head_v_dim;
}

gdn_status check_flags(int32_t flags, int32_t allowed, const int32_t* err_flag) {
    if (flags & ~allowed) return GDN_ERR_FLAGS;
    if ((flags & GDN_FLAG_VALIDATE) && err_flag == nullptr) return GDN_ERR_FLAGS;
    return GDN_OK;
}

#define GDN_TRY_LAUNCH(expr)                                  \
    do {                                                      \
        if ((expr) != hipSuccess) return GDN_ERR_LAUNCH;      \
    } while (0)

}  // namespace

extern "C" {

const char* gdn_strerror(gdn_status s) {
    switch (s) {
        case GDN_OK: return "success";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_DIMS: return "unsupported or inconsistent sizes";
        case GDN_ERR_DTYPE: return "unsupported dtype";
        case GDN_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case GDN_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN_ERR_LAUNCH: return "kernel launch failed";
        case GDN_ERR_FLAGS: return "unknown flag bits, or VALIDATE without err_flag";
    }
    return "unknown status";
}

gdn_status gdn_conv_update(const void* x, gdn_dtype x_dt, const int32_t* cu_seqlens,
                           int32_t n_seqs, int32_t total_tokens, const int32_t* slot_idx,
                           void* conv_state, gdn_dtype cs_dt, int32_t num_slots,
                           const void* weight, const void* bias, gdn_dtype w_dt, void* out,
                           gdn_dtype out_dt, int32_t dim, int32_t width, int32_t flags,
                           int32_t* err_flag, hipStream_t stream) {
    if (gdn_status st = check_flags(flags, GDN_FLAG_SILU | GDN_FLAG_VALIDATE, err_flag)) return st;
    if (n_seqs < 0 || total_tokens < 0 || num_slots < 1 || dim <= 0 || width != 4)
        return GDN_ERR_DIMS;
    if (!cu_seqlens && total_tokens != n_seqs) return GDN_ERR_DIMS;
    if (!cu_seqlens && dim % 4 != 0) return GDN_ERR_DIMS;     // decode form: 4 channels/thread
    if (n_seqs > 65535) return GDN_ERR_DIMS;
    if (!dtype_ok(x_dt) || !dtype_ok(cs_dt) || !dtype_ok(w_dt) || !dtype_ok(out_dt))
        return GDN_ERR_DTYPE;
    if (n_seqs > 0 && (!slot_idx || !conv_state || !weight)) return GDN_ERR_NULL;
    if (total_tokens > 0 && (!x || !out)) return GDN_ERR_NULL;
    if (!cu_seqlens && n_seqs > 0 &&
        (!aligned16(x) || !aligned16(out) || !aligned16(conv_state) || !aligned16(weight) ||
         (bias && !aligned16(bias))))
        return GDN_ERR_ALIGN;
    const hipStream_t s = stream;
    if (flags & GDN_FLAG_VALIDATE)
        GDN_TRY_LAUNCH(launch_validate(slot_idx, n_seqs, num_slots, cu_seqlens, n_seqs, total_tokens,
                                       err_flag, s));
    const int32_t* ef = (flags & GDN_FLAG_VALIDATE) ? err_flag : nullptr;
    if (cu_seqlens)
        GDN_TRY_LAUNCH(launch_conv_varlen(x, x_dt, cu_seqlens, n_seqs, total_tokens, slot_idx,
                                          conv_state, cs_dt, weight, bias, w_dt, out, out_dt, dim,
                                          flags, ef, s));
    else
        GDN_TRY_LAUNCH(launch_conv_decode(x, x_dt, slot_idx, n_seqs, conv_state, cs_dt, weight,
                                          bias, w_dt, out, out_dt, dim, flags, ef, s));
    return GDN_OK;
}

size_t gdn_decode_workspace_size(const gdn_dims* dims, int32_t batch) {
    if (check_dims(dims) != GDN_OK || batch < 0) return 0;
    return round256(static_cast<size_t>(batch) * static_cast<size_t>(conv_channels(dims)) * sizeof(float));
}

int32_t gdn_decode_step_fused(const gdn_dims* dims, int32_t batch) {
    if (check_dims(dims) != GDN_OK || batch < 0 || batch > 65535) return -1;
    return decode_step_use_fused(*dims, batch) ? 1 : 0;
}

}  // extern "C"

namespace {

// The gate source checks shared by the direct and the gated entry points.
gdn_status gate_args(const float* g, const float* beta, const gdn_gate_inputs* gi, bool rows,
                     GateArgs& ga) {
    ga = GateArgs{g, beta, nullptr, nullptr, nullptr, nullptr, 0};
    if (gi) {
        if (!dtype_ok(gi->ab_dt)) return GDN_ERR_DTYPE;
        if (rows && (!gi->a || !gi->b || !gi->A_log || !gi->dt_bias)) return GDN_ERR_NULL;
        ga = GateArgs{nullptr, nullptr, gi->a, gi->b, gi->A_log, gi->dt_bias,
                      gi->ab_dt == GDN_BF16 ? 1 : 0};
        if (!rows) ga.a = nullptr;
    } else if (rows && (!g || !beta)) {
        return GDN_ERR_NULL;
    }
    return GDN_OK;
}

// Scratch of gdn_decode_step_noalloc: the conv + recurrence pair's fp32
// activations live here instead of in a caller workspace.  The array is part
// of the code object, so each device holds its own copy at its own address
// from module load until the process ends; host code must never pass the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// the device address comes from hipGetSymbolAddress, looked up on the first
// call on each device, with that device current, and kept per device.
std::atomic<void*> scratch_addr[64];

void* noalloc_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void* p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        scratch_addr[dev].store(p, std::memory_order_release);   // concurrent first calls agree
    }
    return p;
}

// The decode step's kernels for `batch` rows (after the checks and the
// optional validation): the fused kernel or the conv + recurrence pair.
gdn_status decode_step_launch(const void* mixed_qkv, gdn_dtype x_dt, const GateArgs& ga,
                              const int32_t* slot_idx, int32_t batch, void* conv_state,
                              gdn_dtype cs_dt, const void* conv_weight, const void* conv_bias,
                              gdn_dtype w_dt, float* rec_state, void* out, gdn_dtype out_dt,
                              const gdn_dims* dims, float scale, int32_t flags, void* workspace,
                              const int32_t* ef, hipStream_t s) {
    if (batch == 0) return GDN_OK;
    const int32_t kflags = flags & ~(GDN_FLAG_STEP_FUSED | GDN_FLAG_STEP_SPLIT);
    const bool fused = (flags & GDN_FLAG_STEP_FUSED) ||
                       (!(flags & GDN_FLAG_STEP_SPLIT) && decode_step_use_fused(*dims, batch));
    if (fused) {
        GDN_TRY_LAUNCH(launch_decode_step_fused(mixed_qkv, x_dt, ga, slot_idx, batch, conv_state,
                                                cs_dt, conv_weight, conv_bias, w_dt, rec_state, out,
                                                out_dt, *dims, scale, kflags, ef, s));
        return GDN_OK;
    }
    const int32_t D = static_cast<int32_t>(conv_channels(dims));
    float* y = static_cast<float*>(workspace);
    GDN_TRY_LAUNCH(launch_conv_decode(mixed_qkv, x_dt, slot_idx, batch, conv_state, cs_dt,
                                      conv_weight, conv_bias, w_dt, y, GDN_F32, D,
                                      kflags & GDN_FLAG_SILU, ef, s));
    GDN_TRY_LAUNCH(launch_decode_rec(y, GDN_F32, ga, slot_idx, batch, rec_state, out,
                                     out_dt, *dims, scale, kflags, ef, s));
    return GDN_OK;
}

gdn_status decode_step_impl(const void* mixed_qkv, gdn_dtype x_dt, const float* g,
                            const float* beta, const gdn_gate_inputs* gate,
                            const int32_t* slot_idx, int32_t batch, void* conv_state,
                            gdn_dtype cs_dt, const void* conv_weight, const void* conv_bias,
                            gdn_dtype w_dt, float* rec_state, int32_t num_slots, void* out,
                            gdn_dtype out_dt, const gdn_dims* dims, float scale, int32_t flags,
                            void* workspace, size_t workspace_bytes, int32_t* err_flag,
                            hipStream_t stream, bool use_scratch = false) {
    if (gdn_status st = check_flags(flags, KNOWN_FLAGS | GDN_FLAG_STEP_FUSED | GDN_FLAG_STEP_SPLIT,
                                    err_flag))
        return st;
    if ((flags & GDN_FLAG_STEP_FUSED) && (flags & GDN_FLAG_STEP_SPLIT)) return GDN_ERR_FLAGS;
    if (gdn_status st = check_dims(dims)) return st;
    if (batch < 0 || batch > 65535 || num_slots < 1) return GDN_ERR_DIMS;
    if (static_cast<int64_t>(batch) * dims->num_v_heads > (1 << 24)) return GDN_ERR_DIMS;
    if ((flags & GDN_FLAG_STEP_FUSED) && !decode_step_fused_fits(*dims)) return GDN_ERR_DIMS;
    if (!dtype_ok(x_dt) || !dtype_ok(cs_dt) || !dtype_ok(w_dt) || !dtype_ok(out_dt))
        return GDN_ERR_DTYPE;
    GateArgs ga;
    if (gdn_status st = gate_args(g, beta, gate, batch > 0, ga)) return st;
    if (batch > 0) {
        if (!mixed_qkv || !slot_idx || !conv_state || !conv_weight || !rec_state || !out ||
            (!workspace && !use_scratch))
            return GDN_ERR_NULL;
        if (!aligned16(rec_state) || !aligned16(workspace) || !aligned16(mixed_qkv) ||
            !aligned16(conv_state) || !aligned16(conv_weight) || (conv_bias && !aligned16(conv_bias)))
            return GDN_ERR_ALIGN;
        if (use_scratch) {
            // the library's scratch array stands in for the workspace; it is
            // needed only when the call takes the conv + recurrence pair (the
            // fused kernel keeps the activations in LDS).  Where the pair's
            // activations would not fit, the default path takes the fused
            // kernel instead (the same bits); a forced pair is rejected.
            const bool fused = (flags & GDN_FLAG_STEP_FUSED) ||
                               (!(flags & GDN_FLAG_STEP_SPLIT) && decode_step_use_fused(*dims, batch));
            if (!fused && gdn_decode_workspace_size(dims, batch) > GDN_NOALLOC_SCRATCH_BYTES) {
                if ((flags & GDN_FLAG_STEP_SPLIT) || !decode_step_fused_fits(*dims))
                    return GDN_ERR_WORKSPACE;
                flags |= GDN_FLAG_STEP_FUSED;
            }
            workspace = noalloc_scratch();
            if (!workspace) return GDN_ERR_LAUNCH;
        } else if (workspace_bytes < gdn_decode_workspace_size(dims, batch)) {
            return GDN_ERR_WORKSPACE;
        }
    }
    const hipStream_t s = stream;
    if (flags & GDN_FLAG_VALIDATE)
        GDN_TRY_LAUNCH(launch_validate(slot_idx, batch, num_slots, nullptr, 0, 0, err_flag, s));
    const int32_t* ef = (flags & GDN_FLAG_VALIDATE) ? err_flag : nullptr;
    return decode_step_launch(mixed_qkv, x_dt, ga, slot_idx, batch, conv_state, cs_dt, conv_weight,
                              conv_bias, w_dt, rec_state, out, out_dt, dims, scale, flags,
                              workspace, ef, s);
}

gdn_status prefill_impl(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                        const float* g, const float* beta, const gdn_gate_inputs* gate,
                        const int32_t* cu_seqlens, int32_t n_seqs, int32_t total_tokens,
                        const int32_t* slot_idx, float* rec_state, int32_t num_slots, void* out,
                        gdn_dtype out_dt, const gdn_dims* dims, float scale, int32_t flags,
                        int32_t seg_len, int32_t head_len, void* workspace,
                        size_t workspace_bytes, int32_t* err_flag, hipStream_t stream) {
    if (gdn_status st = check_flags(flags, GDN_FLAG_QK_L2NORM | GDN_FLAG_VALIDATE |
                                               GDN_FLAG_PREFILL_NS3 | GDN_FLAG_PREFILL_NS4 |
                                               GDN_FLAG_PREFILL_SEQUENTIAL |
                                               GDN_FLAG_PREFILL_SINGLE_ROLE,
                                    err_flag))
        return st;
    if ((flags & GDN_FLAG_PREFILL_NS3) && (flags & GDN_FLAG_PREFILL_NS4)) return GDN_ERR_FLAGS;
    if (gdn_status st = check_dims(dims)) return st;
    if (n_seqs < 0 || n_seqs > 65535 || total_tokens < 0 || num_slots < 1) return GDN_ERR_DIMS;
    if (!dtype_ok(in_dt) || !dtype_ok(out_dt)) return GDN_ERR_DTYPE;
    if (dims->head_k_dim != dims->head_v_dim || dims->head_k_dim > 128) return GDN_ERR_DIMS;
    if (!prefill_supported(*dims, in_dt)) return GDN_ERR_DTYPE;
    GateArgs ga;
    if (gdn_status st = gate_args(g, beta, gate, total_tokens > 0, ga)) return st;
    if (n_seqs > 0 && (!cu_seqlens || !slot_idx || !rec_state)) return GDN_ERR_NULL;
    if (total_tokens > 0 && (!q || !k || !v || !out)) return GDN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(rec_state))
        return GDN_ERR_ALIGN;
    PrefillSchedule sch{0, 0, true};
    if (seg_len > 0) {                           // explicit segment lengths
        if (seg_len % 64 != 0) return GDN_ERR_DIMS;
        if (head_len == 0) head_len = seg_len;
        if (head_len < seg_len || head_len % 64 != 0) return GDN_ERR_DIMS;
        // at head dim 128 a middle segment's P and B runs are workgroups of
        // their own on the pipelined step (faster than the paired single-role
        // workgroup there); at 32 and 64 they share one
        sch = PrefillSchedule{seg_len, head_len, dims->head_k_dim < 128};
        if (flags & GDN_FLAG_PREFILL_SEQUENTIAL) return GDN_ERR_FLAGS;
        if ((total_tokens + seg_len - 1) / seg_len > 32768) return GDN_ERR_DIMS;
        if (!prefill_seg_grid_fits(n_seqs, total_tokens, sch)) return GDN_ERR_DIMS;
        if (n_seqs > 0 && total_tokens > 0) {
            if (!workspace) return GDN_ERR_WORKSPACE;
            if (workspace_bytes < prefill_segmented_workspace(*dims, n_seqs, total_tokens, seg_len))
                return GDN_ERR_WORKSPACE;
            if (!aligned16(workspace)) return GDN_ERR_ALIGN;
        }
    } else if (seg_len < 0) {                    // the plain call: segments when they pay
        if (!(flags & GDN_FLAG_PREFILL_SEQUENTIAL)) sch = prefill_auto_schedule(*dims, n_seqs, total_tokens);
        if (sch.seg_len > 0 &&
            (!workspace || !aligned16(workspace) ||
             workspace_bytes < prefill_segmented_workspace(*dims, n_seqs, total_tokens, sch.seg_len)))
            sch = PrefillSchedule{0, 0, true};
    } else {
        return GDN_ERR_DIMS;
    }
    const hipStream_t s = stream;
    if (flags & GDN_FLAG_VALIDATE)
        GDN_TRY_LAUNCH(launch_validate(slot_idx, n_seqs, num_slots, cu_seqlens, n_seqs, total_tokens,
                                       err_flag, s));
    const int32_t* ef = (flags & GDN_FLAG_VALIDATE) ? err_flag : nullptr;
    const int32_t sqk = dims->num_k_heads * dims->head_k_dim;
    const int32_t sv = dims->num_v_heads * dims->head_v_dim;
    if (sch.seg_len > 0 && n_seqs > 0 && total_tokens > 0)
        GDN_TRY_LAUNCH(launch_prefill_segmented(q, k, v, in_dt, ga, cu_seqlens, n_seqs,
                                                total_tokens, slot_idx, rec_state, out, out_dt,
                                                *dims, sqk, sv, scale, flags, sch,
                                                static_cast<float*>(workspace), ef, s));
    else
        GDN_TRY_LAUNCH(launch_prefill(q, k, v, in_dt, ga, cu_seqlens, n_seqs, slot_idx,
                                      rec_state, out, out_dt, *dims, sqk, sv, scale, flags, ef, s));
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_decode_step(const void* mixed_qkv, gdn_dtype x_dt, const float* g,
                           const float* beta, const int32_t* slot_idx, int32_t batch,
                           void* conv_state, gdn_dtype cs_dt, const void* conv_weight,
                           const void* conv_bias, gdn_dtype w_dt, float* rec_state,
                           int32_t num_slots, void* out, gdn_dtype out_dt, const gdn_dims* dims,
                           float scale, int32_t flags, void* workspace, size_t workspace_bytes,
                           int32_t* err_flag, hipStream_t stream) {
    return decode_step_impl(mixed_qkv, x_dt, g, beta, nullptr, slot_idx, batch, conv_state,
                            cs_dt, conv_weight, conv_bias, w_dt, rec_state, num_slots, out,
                            out_dt, dims, scale, flags, workspace, workspace_bytes, err_flag,
                            stream);
}

gdn_status gdn_decode_step_gated(const void* mixed_qkv, gdn_dtype x_dt,
                                 const gdn_gate_inputs* gate, const int32_t* slot_idx,
                                 int32_t batch, void* conv_state, gdn_dtype cs_dt,
                                 const void* conv_weight, const void* conv_bias, gdn_dtype w_dt,
                                 float* rec_state, int32_t num_slots, void* out, gdn_dtype out_dt,
                                 const gdn_dims* dims, float scale, int32_t flags,
                                 void* workspace, size_t workspace_bytes, int32_t* err_flag,
                                 hipStream_t stream) {
    if (!gate) return GDN_ERR_NULL;
    return decode_step_impl(mixed_qkv, x_dt, nullptr, nullptr, gate, slot_idx, batch,
                            conv_state, cs_dt, conv_weight, conv_bias, w_dt, rec_state,
                            num_slots, out, out_dt, dims, scale, flags, workspace,
                            workspace_bytes, err_flag, stream);
}

gdn_status gdn_decode_step_noalloc(const void* mixed_qkv, gdn_dtype x_dt, const float* g,
                                   const float* beta, const int32_t* slot_idx, int32_t batch,
                                   void* conv_state, gdn_dtype cs_dt, const void* conv_weight,
                                   const void* conv_bias, gdn_dtype w_dt, float* rec_state,
                                   int32_t num_slots, void* out, gdn_dtype out_dt,
                                   const gdn_dims* dims, float scale, int32_t flags,
                                   int32_t* err_flag, hipStream_t stream) {
    return decode_step_impl(mixed_qkv, x_dt, g, beta, nullptr, slot_idx, batch, conv_state,
                            cs_dt, conv_weight, conv_bias, w_dt, rec_state, num_slots, out,
                            out_dt, dims, scale, flags, nullptr, 0, err_flag, stream, true);
}

gdn_status gdn_decode_recurrent(const void* qkv, gdn_dtype qkv_dt, const float* g,
                                const float* beta, const int32_t* slot_idx, int32_t batch,
                                float* rec_state, int32_t num_slots, void* out, gdn_dtype out_dt,
                                const gdn_dims* dims, float scale, int32_t flags,
                                int32_t* err_flag, hipStream_t stream) {
    if (gdn_status st = check_flags(flags, GDN_FLAG_QK_L2NORM | GDN_FLAG_VALIDATE, err_flag))
        return st;
    if (gdn_status st = check_dims(dims)) return st;
    if (batch < 0 || batch > 65535 || num_slots < 1) return GDN_ERR_DIMS;
    if (static_cast<int64_t>(batch) * dims->num_v_heads > (1 << 24)) return GDN_ERR_DIMS;
    if (!dtype_ok(qkv_dt) || !dtype_ok(out_dt)) return GDN_ERR_DTYPE;
    GateArgs ga;
    if (gdn_status st = gate_args(g, beta, nullptr, batch > 0, ga)) return st;
    if (batch > 0) {
        if (!qkv || !slot_idx || !rec_state || !out) return GDN_ERR_NULL;
        if (!aligned16(rec_state) || !aligned16(qkv)) return GDN_ERR_ALIGN;
    }
    const hipStream_t s = stream;
    if (flags & GDN_FLAG_VALIDATE)
        GDN_TRY_LAUNCH(launch_validate(slot_idx, batch, num_slots, nullptr, 0, 0, err_flag, s));
    const int32_t* ef = (flags & GDN_FLAG_VALIDATE) ? err_flag : nullptr;
    GDN_TRY_LAUNCH(launch_decode_rec(qkv, qkv_dt, ga, slot_idx, batch, rec_state, out,
                                     out_dt, *dims, scale, flags, ef, s));
    return GDN_OK;
}

size_t gdn_prefill_workspace_size(const gdn_dims* dims, int32_t n_seqs, int32_t total_tokens) {
    // Whole-sequence runs keep every intermediate on chip; the segment-parallel
    // schedule, where the call would choose it, needs its segment matrices.
    if (check_dims(dims) != GDN_OK || n_seqs <= 0 || total_tokens <= 0) return 0;
    if (dims->head_k_dim != dims->head_v_dim || dims->head_k_dim > 128) return 0;
    return prefill_segmented_workspace(*dims, n_seqs, total_tokens,
                                       prefill_auto_schedule(*dims, n_seqs, total_tokens).seg_len);
}

size_t gdn_prefill_segmented_workspace_size(const gdn_dims* dims, int32_t n_seqs,
                                            int32_t total_tokens, int32_t seg_len) {
    if (check_dims(dims) != GDN_OK || n_seqs < 0 || total_tokens < 0) return 0;
    if (seg_len <= 0 || seg_len % 64 != 0) return 0;
    if (dims->head_k_dim != dims->head_v_dim || dims->head_k_dim > 128) return 0;
    return prefill_segmented_workspace(*dims, n_seqs, total_tokens, seg_len);
}

gdn_status gdn_prefill_segmented(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                                 const float* g, const float* beta, const gdn_gate_inputs* gate,
                                 const int32_t* cu_seqlens, int32_t n_seqs, int32_t total_tokens,
                                 const int32_t* slot_idx, float* rec_state, int32_t num_slots,
                                 void* out, gdn_dtype out_dt, const gdn_dims* dims, float scale,
                                 int32_t flags, int32_t seg_len, int32_t head_len,
                                 void* workspace, size_t workspace_bytes, int32_t* err_flag,
                                 hipStream_t stream) {
    if (seg_len <= 0 || head_len < 0) return GDN_ERR_DIMS;
    if (gate && (g || beta)) return GDN_ERR_FLAGS;
    return prefill_impl(q, k, v, in_dt, gate ? nullptr : g, gate ? nullptr : beta, gate,
                        cu_seqlens, n_seqs, total_tokens, slot_idx, rec_state, num_slots, out,
                        out_dt, dims, scale, flags, seg_len, head_len, workspace,
                        workspace_bytes, err_flag, stream);
}

gdn_status gdn_prefill_chunked(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                               const float* g, const float* beta, const int32_t* cu_seqlens,
                               int32_t n_seqs, int32_t total_tokens, const int32_t* slot_idx,
                               float* rec_state, int32_t num_slots, void* out, gdn_dtype out_dt,
                               const gdn_dims* dims, float scale, int32_t flags, void* workspace,
                               size_t workspace_bytes, int32_t* err_flag, hipStream_t stream) {
    return prefill_impl(q, k, v, in_dt, g, beta, nullptr, cu_seqlens, n_seqs, total_tokens,
                        slot_idx, rec_state, num_slots, out, out_dt, dims, scale, flags, -1, 0,
                        workspace, workspace_bytes, err_flag, stream);
}

gdn_status gdn_prefill_chunked_gated(const void* q, const void* k, const void* v,
                                     gdn_dtype in_dt, const gdn_gate_inputs* gate,
                                     const int32_t* cu_seqlens, int32_t n_seqs,
                                     int32_t total_tokens, const int32_t* slot_idx,
                                     float* rec_state, int32_t num_slots, void* out,
                                     gdn_dtype out_dt, const gdn_dims* dims, float scale,
                                     int32_t flags, void* workspace, size_t workspace_bytes,
                                     int32_t* err_flag, hipStream_t stream) {
    if (!gate) return GDN_ERR_NULL;
    return prefill_impl(q, k, v, in_dt, nullptr, nullptr, gate, cu_seqlens, n_seqs,
                        total_tokens, slot_idx, rec_state, num_slots, out, out_dt, dims, scale,
                        flags, -1, 0, workspace, workspace_bytes, err_flag, stream);
}

size_t gdn_mixed_workspace_size(const gdn_dims* dims, int32_t n_dec, int32_t total_pre) {
    if (check_dims(dims) != GDN_OK || n_dec < 0 || total_pre < 0) return 0;
    const size_t D = static_cast<size_t>(conv_channels(dims));
    return round256(static_cast<size_t>(n_dec) * D * sizeof(float)) +
           round256(static_cast<size_t>(total_pre) * D * sizeof(uint16_t));
}

gdn_status gdn_mixed_step(const void* x, gdn_dtype x_dt, const float* g, const float* beta,
                          int32_t n_dec, const int32_t* cu_seqlens, int32_t n_pre,
                          int32_t total_pre, const int32_t* slot_idx, void* conv_state,
                          gdn_dtype cs_dt, const void* conv_weight, const void* conv_bias,
                          gdn_dtype w_dt, float* rec_state, int32_t num_slots, void* out,
                          gdn_dtype out_dt, const gdn_dims* dims, float scale, int32_t flags,
                          void* workspace, size_t workspace_bytes, int32_t* err_flag,
                          hipStream_t stream, hipStream_t prefill_stream, hipEvent_t fork_event,
                          hipEvent_t join_event) {
    if (gdn_status st = check_flags(flags, KNOWN_FLAGS | GDN_FLAG_STEP_FUSED | GDN_FLAG_STEP_SPLIT |
                                               GDN_FLAG_PREFILL_SEQUENTIAL |
                                               GDN_FLAG_PREFILL_SINGLE_ROLE,
                                    err_flag))
        return st;
    if ((flags & GDN_FLAG_STEP_FUSED) && (flags & GDN_FLAG_STEP_SPLIT)) return GDN_ERR_FLAGS;
    if (gdn_status st = check_dims(dims)) return st;
    if (n_dec < 0 || n_pre < 0 || total_pre < 0 || num_slots < 1) return GDN_ERR_DIMS;
    if (static_cast<int64_t>(n_dec) + n_pre > 65535) return GDN_ERR_DIMS;
    if (static_cast<int64_t>(n_dec) * dims->num_v_heads > (1 << 24)) return GDN_ERR_DIMS;
    if (static_cast<int64_t>(n_dec) + total_pre > (1LL << 31) - 1) return GDN_ERR_DIMS;
    if ((flags & GDN_FLAG_STEP_FUSED) && !decode_step_fused_fits(*dims)) return GDN_ERR_DIMS;
    if (n_pre > 0 && (dims->head_k_dim != dims->head_v_dim || dims->head_k_dim > 128 ||
                      !prefill_supported(*dims, GDN_BF16)))
        return GDN_ERR_DIMS;
    if (!dtype_ok(x_dt) || !dtype_ok(cs_dt) || !dtype_ok(w_dt) || !dtype_ok(out_dt))
        return GDN_ERR_DTYPE;
    const int64_t rows = static_cast<int64_t>(n_dec) + total_pre;
    GateArgs ga;
    if (gdn_status st = gate_args(g, beta, nullptr, rows > 0, ga)) return st;
    if (n_dec + n_pre > 0 && (!slot_idx || !conv_state || !conv_weight || !rec_state))
        return GDN_ERR_NULL;
    if (n_pre > 0 && !cu_seqlens) return GDN_ERR_NULL;
    if (rows > 0 && (!x || !out || !workspace)) return GDN_ERR_NULL;
    if (!aligned16(x) || !aligned16(rec_state) || !aligned16(workspace) || !aligned16(conv_state) ||
        !aligned16(conv_weight) || (conv_bias && !aligned16(conv_bias)))
        return GDN_ERR_ALIGN;
    if (rows > 0 && workspace_bytes < gdn_mixed_workspace_size(dims, n_dec, total_pre))
        return GDN_ERR_WORKSPACE;
    if (prefill_stream && (!fork_event || !join_event)) return GDN_ERR_NULL;
    const hipStream_t s = stream;
    if (flags & GDN_FLAG_VALIDATE)
        GDN_TRY_LAUNCH(launch_validate(slot_idx, n_dec + n_pre, num_slots, n_pre > 0 ? cu_seqlens : nullptr,
                                       n_pre, total_pre, err_flag, s));
    const int32_t* ef = (flags & GDN_FLAG_VALIDATE) ? err_flag : nullptr;
    const int32_t D = static_cast<int32_t>(conv_channels(dims));
    const int32_t HV = dims->num_v_heads, dv = dims->head_v_dim;
    const size_t esx = (x_dt == GDN_BF16) ? 2 : 4;
    const size_t eso = (out_dt == GDN_BF16) ? 2 : 4;

    // decode rows: the decode-only step's kernels (rows 0 .. n_dec-1).  Beside
    // a prefill part on its own stream they take the fused kernel where it
    // fits (the same bits as the pair): one 1024-thread group per CU lets the
    // prefill's workgroups take CUs as the groups retire, while the pair's
    // small recurrence workgroups keep every CU busy to the end (256 decode
    // rows + 2 x 1024 prefill tokens: 0.247 ms fused, 0.309 ms with the pair).
    auto decode_part = [&](hipStream_t ds, bool overlapped) -> gdn_status {
        int32_t df = flags;
        if (overlapped && !(flags & GDN_FLAG_STEP_SPLIT) && decode_step_fused_fits(*dims) &&
            dims->head_k_dim <= 128)
            df |= GDN_FLAG_STEP_FUSED;
        return decode_step_launch(x, x_dt, ga, slot_idx, n_dec, conv_state, cs_dt, conv_weight, conv_bias,
                                  w_dt, rec_state, out, out_dt, dims, scale, df, workspace, ef, ds);
    };
    // prefill tokens (rows n_dec ..): varlen conv into bf16 activations, then
    // the chunked prefill reading q, k, v as slices of those rows
    auto prefill_part = [&](hipStream_t ps, bool beside_decode) -> gdn_status {
        const char* xp = static_cast<const char*>(x) + static_cast<size_t>(n_dec) * D * esx;
        uint16_t* yp = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) +
                                               round256(static_cast<size_t>(n_dec) * D * sizeof(float)));
        const int32_t* sp = slot_idx + n_dec;
        GDN_TRY_LAUNCH(launch_conv_varlen(xp, x_dt, cu_seqlens, n_pre, total_pre, sp, conv_state,
                                          cs_dt, conv_weight, conv_bias, w_dt, yp, GDN_BF16, D,
                                          flags & GDN_FLAG_SILU, ef, ps));
        GateArgs gp = ga;
        gp.g = ga.g + static_cast<size_t>(n_dec) * HV;
        gp.beta = ga.beta + static_cast<size_t>(n_dec) * HV;
        const int32_t Hdk = dims->num_k_heads * dims->head_k_dim;
        void* op = static_cast<char*>(out) + static_cast<size_t>(n_dec) * HV * dv * eso;
        // the segment-parallel schedule that gdn_prefill_chunked would pick, when
        // the workspace holds its segment states past the activations -- but not
        // beside decode rows: there the CUs it would fill are the decode's, and
        // whole runs overlapped with the decode measured faster.  The choice
        // depends on the call's arguments only (never on the streams given).
        const size_t base = gdn_mixed_workspace_size(dims, n_dec, total_pre);
        PrefillSchedule sch{0, 0, true};
        if (!(flags & GDN_FLAG_PREFILL_SEQUENTIAL) && !beside_decode)
            sch = prefill_auto_schedule(*dims, n_pre, total_pre);
        if (sch.seg_len > 0 &&
            workspace_bytes - base < prefill_segmented_workspace(*dims, n_pre, total_pre, sch.seg_len))
            sch = PrefillSchedule{0, 0, true};
        if (sch.seg_len > 0)
            GDN_TRY_LAUNCH(launch_prefill_segmented(yp, yp + Hdk, yp + 2 * Hdk, GDN_BF16, gp, cu_seqlens,
                                                    n_pre, total_pre, sp, rec_state, op, out_dt, *dims,
                                                    D, D, scale, flags & (GDN_FLAG_QK_L2NORM | GDN_FLAG_PREFILL_SINGLE_ROLE), sch,
                                                    reinterpret_cast<float*>(static_cast<char*>(workspace) + base),
                                                    ef, ps));
        else
            GDN_TRY_LAUNCH(launch_prefill(yp, yp + Hdk, yp + 2 * Hdk, GDN_BF16, gp, cu_seqlens, n_pre, sp,
                                          rec_state, op, out_dt, *dims, D, D, scale,
                                          flags & (GDN_FLAG_QK_L2NORM | GDN_FLAG_PREFILL_SINGLE_ROLE), ef, ps));
        return GDN_OK;
    };
    // sequences without tokens leave their state untouched: nothing to launch
    const bool has_pre = n_pre > 0 && total_pre > 0;
    const bool beside = has_pre && n_dec > 0;
    if (!beside || !prefill_stream) {
        if (gdn_status st = decode_part(s, false)) return st;
        return has_pre ? prefill_part(s, beside) : GDN_OK;
    }
    // The two parts touch disjoint rows, slots and workspace regions, and a CU
    // cannot hold a workgroup of each, so the prefill runs on the caller's
    // prefill_stream (forked from `stream` after the validation and joined
    // back into it by the caller's events) and takes CUs as the decode's
    // workgroups retire.  The join is enqueued even after a failed launch, so
    // `stream` stays ordered after everything this call enqueued.
    if (hipEventRecord(fork_event, s) != hipSuccess ||
        hipStreamWaitEvent(prefill_stream, fork_event, 0) != hipSuccess)
        return GDN_ERR_LAUNCH;
    const gdn_status sp_st = prefill_part(prefill_stream, true);
    const gdn_status sd_st = sp_st == GDN_OK ? decode_part(s, true) : GDN_OK;
    const bool joined = hipEventRecord(join_event, prefill_stream) == hipSuccess &&
                        hipStreamWaitEvent(s, join_event, 0) == hipSuccess;
    if (sp_st != GDN_OK) return sp_st;
    if (sd_st != GDN_OK) return sd_st;
    return joined ? GDN_OK : GDN_ERR_LAUNCH;
}

gdn_status gdn_gated_rmsnorm(const void* x, gdn_dtype x_dt, const void* z, const void* weight,
                             gdn_dtype w_dt, int64_t rows, int32_t dim, float eps, int32_t flags,
                             void* out, gdn_dtype out_dt, hipStream_t stream) {
    if (flags & ~(GDN_NORM_GATE_SIGMOID | GDN_NORM_ZERO_CENTRED)) return GDN_ERR_FLAGS;
    if (rows < 0 || dim < 4 || dim > 1024 || dim % 4 != 0 || !(eps >= 0.0f)) return GDN_ERR_DIMS;
    if (rows > (static_cast<int64_t>(1) << 32)) return GDN_ERR_DIMS;
    if (!dtype_ok(x_dt) || !dtype_ok(w_dt) || !dtype_ok(out_dt)) return GDN_ERR_DTYPE;
    if (rows > 0 && (!x || !weight || !out)) return GDN_ERR_NULL;
    if (!aligned16(x) || !aligned16(weight) || !aligned16(out) || (z && !aligned16(z)))
        return GDN_ERR_ALIGN;
    GDN_TRY_LAUNCH(launch_gated_rmsnorm(x, x_dt, z, weight, w_dt, out, out_dt, rows, dim, eps,
                                        flags, stream));
    return GDN_OK;
}

}  // extern "C"
