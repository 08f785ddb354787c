// decode.hip -- gated delta-rule decode update of a slot-indexed fp32 state.
//
// Per active row b and value head hv (key head h = hv / (HV / H), RL-Kernel
// PR #469, "How the golden relates to the kernel", item 2):
//   q, k  <- post-conv activations, L2-normalised x / sqrt(sum(x*x) + 1e-6),
//            q multiplied by `scale` after the norm, k never scaled (item 3)
//   alpha = exp(g);  S1 = alpha * S;  u = S1 k;  S' = S1 + beta (v - u) k^T;
//   o = S' q;  S' stored back in fp32 (RL-Kernel PR #469, "Summary": the
//   state is [num_blocks, HV, V, K], fp32 accumulator, the store rounds to the
//   state dtype -- fp32 here).
//
// The kernel is a stream of the fp32 state (2 MiB read + 2 MiB written per
// sequence at HV = 32, d = 128), so it is HBM-bound.  Layout in registers:
// a state row S[v, :] (dk floats, contiguous) is spread over 8 lanes; lane
// `sub` of the group holds the float4s at k = 32 i + 4 sub (i < dk / 32), so
// each load instruction of a wave covers 8 full 128-byte lines.  A wave holds
// 8 rows per step; a 256-thread workgroup holds 32 rows per step and RPL
// steps, i.e. 32 * RPL rows of one (row, head).  Each lane issues every load
// of its rows before any arithmetic, so 256 * 16 * RPL * dk / 32 bytes are in
// flight per workgroup.  Both row reductions (S1 k and S' q) are an in-lane
// fixed-order fma chain followed by the 8-lane DPP butterfly `sum8`: the order
// depends on nothing but dk, so results are batch-invariant and replay
// bitwise.  No LDS is used at all.

#include "conv_io.hpp"
#include "gate.hpp"
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

// Four consecutive activations as fp32 (16-byte load for fp32, 8 for bf16).
template <typename YT> __device__ __forceinline__ float4 load4(const YT* p);
template <> __device__ __forceinline__ float4 load4<float>(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
template <> __device__ __forceinline__ float4 load4<bf16_t>(const bf16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

// Workgroups per CU in the recurrence kernel's grid (an item-strided loop
// beyond it), and whether the state stream uses nontemporal loads/stores (it
// is read once and written once).  One workgroup per 32-row item up to batch
// 1024 at HV = 32: the hardware then starts an item's loads as soon as a
// workgroup slot frees, which a loop over items inside a resident workgroup
// does not (batch 256, 32768 items: 16 per CU, eight items per workgroup,
// 191.8 us; 64 per CU 181.2 us; 128, one item each, 174.9 us = 6.2 TB/s;
// batch 1024: 807 / 784 / 764 us, and the whole step 785 us at 512).
#ifndef GDN_DECODE_WG_PER_CU
#define GDN_DECODE_WG_PER_CU 512
#endif
#ifndef GDN_DECODE_NT
#define GDN_DECODE_NT 1
#endif
// Largest rows-per-lane step count (a workgroup item covers 32 x RPL rows).
// Small items (32 rows, 16 KB of state) measured fastest: the workgroups in
// flight then stream a narrower window of the cache.
#ifndef GDN_DECODE_RPL_MAX
#define GDN_DECODE_RPL_MAX 1
#endif

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 state_ld(const float* p) {
#if GDN_DECODE_NT
    const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
#else
    return *reinterpret_cast<const float4*>(p);
#endif
}
__device__ __forceinline__ void state_st(float* p, const float4& x) {
#if GDN_DECODE_NT
    const v4f v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(p));
#else
    *reinterpret_cast<float4*>(p) = x;
#endif
}

template <int DK, int RPL, bool FULL, bool GATED, typename YT, typename OT>
__device__ __forceinline__ void rec_item(
    const YT* __restrict__ y, const GateArgs& ga,
    const int32_t* __restrict__ slot, float* __restrict__ rec, OT* __restrict__ out, int32_t H,
    int32_t HV, int32_t dv, int b, int hv, int tile, float scale, int32_t flags) {
    constexpr int NV = DK / 32;               // float4 per lane per row
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane & 7;
    const int row0 = tile * (32 * RPL) + wave * 8 + (lane >> 3);   // + 32 r
    const int32_t s = slot[b];
    OT* ob = out + (static_cast<size_t>(b) * HV + hv) * dv;

    if (s <= 0) {                             // inactive row: zeros, state untouched
        if (sub == 0) {
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                const int row = row0 + 32 * r;
                if (FULL || row < dv) elem<OT>::st(ob + row, 0.0f);
            }
        }
        return;                               // next item
    }

    // 0. fused gating: its inputs first, so their (in-order) wait never waits
    //    for the state
    float gx0 = 0.0f, gx1 = 0.0f;
    GateHead gh{0.0f, 0.0f};
    if constexpr (GATED) {
        gate_raw(ga, static_cast<size_t>(b) * HV + hv, gx0, gx1);
        gh = gate_head(ga, hv);
    }

    const int D = 2 * H * DK + HV * dv;
    const int h = hv / (HV / H);
    const YT* yb = y + static_cast<size_t>(b) * D;
    float* Sb = rec + (static_cast<size_t>(s) * HV + hv) * static_cast<size_t>(dv) * DK;

    // 1. q, k fragments of key head h first (small, L2-resident activations)
    float4 qf[NV], kf[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        qf[i] = load4<YT>(yb + h * DK + 32 * i + 4 * sub);
        kf[i] = load4<YT>(yb + H * DK + h * DK + 32 * i + 4 * sub);
    }
    const YT* vb = yb + 2 * H * DK + hv * dv;
    float vv[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int row = row0 + 32 * r;
        vv[r] = (FULL || row < dv) ? elem<YT>::ld(vb + row) : 0.0f;
    }
    // 2. then the state loads (the long-latency HBM stream): with full tiles
    //    (no row guards) the norm math below waits only for q, k and v, and
    //    each row only for its own loads
    float4 S[RPL][NV];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int row = row0 + 32 * r;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            S[r][i] = (FULL || row < dv) ? state_ld(Sb + static_cast<size_t>(row) * DK + 32 * i + 4 * sub)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    float qmul = scale, kmul = 1.0f;
    if (flags & GDN_FLAG_QK_L2NORM) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            sq = fmaf(qf[i].x, qf[i].x, sq); sq = fmaf(qf[i].y, qf[i].y, sq);
            sq = fmaf(qf[i].z, qf[i].z, sq); sq = fmaf(qf[i].w, qf[i].w, sq);
            sk = fmaf(kf[i].x, kf[i].x, sk); sk = fmaf(kf[i].y, kf[i].y, sk);
            sk = fmaf(kf[i].z, kf[i].z, sk); sk = fmaf(kf[i].w, kf[i].w, sk);
        }
        sq = sum8(sq);
        sk = sum8(sk);
        qmul = scale / sqrtf(sq + 1e-6f);
        kmul = 1.0f / sqrtf(sk + 1e-6f);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        qf[i].x *= qmul; qf[i].y *= qmul; qf[i].z *= qmul; qf[i].w *= qmul;
        kf[i].x *= kmul; kf[i].y *= kmul; kf[i].z *= kmul; kf[i].w *= kmul;
    }

    float gv, bt;
    if constexpr (GATED) {
        gate_finish(ga, gh, gx0, gx1, gv, bt);
    } else {
        gv = ga.g[static_cast<size_t>(b) * HV + hv];
        bt = ga.beta[static_cast<size_t>(b) * HV + hv];
    }
    const float alpha = expf(gv);

    // 3. per row: decay, predict, delta update, output
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const int row = row0 + 32 * r;
        float u = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            S[r][i].x *= alpha; S[r][i].y *= alpha; S[r][i].z *= alpha; S[r][i].w *= alpha;
            u = fmaf(S[r][i].x, kf[i].x, u); u = fmaf(S[r][i].y, kf[i].y, u);
            u = fmaf(S[r][i].z, kf[i].z, u); u = fmaf(S[r][i].w, kf[i].w, u);
        }
        u = sum8(u);
        const float delta = bt * (vv[r] - u);
        float o = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            S[r][i].x = fmaf(delta, kf[i].x, S[r][i].x); S[r][i].y = fmaf(delta, kf[i].y, S[r][i].y);
            S[r][i].z = fmaf(delta, kf[i].z, S[r][i].z); S[r][i].w = fmaf(delta, kf[i].w, S[r][i].w);
            o = fmaf(S[r][i].x, qf[i].x, o); o = fmaf(S[r][i].y, qf[i].y, o);
            o = fmaf(S[r][i].z, qf[i].z, o); o = fmaf(S[r][i].w, qf[i].w, o);
        }
        o = sum8(o);
        if (FULL || row < dv) {
#pragma unroll
            for (int i = 0; i < NV; ++i)
                state_st(Sb + static_cast<size_t>(row) * DK + 32 * i + 4 * sub, S[r][i]);
            if (sub == 0) elem<OT>::st(ob + row, o);
        }
    }
}

template <int DK, int RPL, bool FULL, bool GATED, typename YT, typename OT>
__global__ __launch_bounds__(256) void decode_rec_kernel(
    const YT* __restrict__ y, const GateArgs ga,
    const int32_t* __restrict__ slot, float* __restrict__ rec, OT* __restrict__ out, int32_t H,
    int32_t HV, int32_t dv, int32_t tiles_per_head, int32_t n_items, float scale,
    int32_t flags, const int32_t* __restrict__ err_flag) {
    constexpr int NV = DK / 32;               // float4 per lane per row
    if (call_rejected(err_flag)) return;
    // one (row, value head, tile) item per workgroup up to the grid's cap, a
    // workgroup-uniform loop over items beyond it
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int per_row = HV * tiles_per_head;
        const int b = item / per_row;
        const int hv = (item - b * per_row) / tiles_per_head;
        const int tile = item - b * per_row - hv * tiles_per_head;
        rec_item<DK, RPL, FULL, GATED, YT, OT>(y, ga, slot, rec, out, H, HV, dv, b, hv, tile, scale, flags);
    }
}

// ---------------------------------------------------------------------------
// Fused decode step.  One workgroup per (row b, key head h) group owns the
// group's conv channels -- q_h, k_h and the v channels of the G = HV / H value
// heads that share h -- so it reads and rolls them with no other workgroup
// touching them, and keeps the post-conv activations in LDS instead of an HBM
// workspace.  The recurrence then streams the group's G dv state rows in
// passes of NT / 8 rows with the per-row arithmetic of rec_item, in the same
// order, so this kernel and the conv kernel + decode_rec_kernel pair give
// bitwise-identical results.  The first pass's state loads are issued right
// after the conv's own loads, so that they are in flight during the conv.
//
// DB (double-buffered passes): the second pass's loads also go out before the
// conv, and each pass's loads go out as soon as the pass two back has stored,
// so one pass computes while the next one streams in.  q is re-read from LDS
// in each row (and scaled there) to keep the 16 extra state registers well
// under the 128-register cap of 1024-thread groups (111-113 VGPRs; 127 with q in
// registers, measured no faster).  With one or two groups per CU the step is a
// short latency chain per CU, and there double-buffering saves 15% (batch 16);
// with many groups queued per CU it costs 1.5-2% (batch 256), q placement aside.
// ---------------------------------------------------------------------------
// Threads per fused-step workgroup: a pass streams NT / 8 state rows.
#ifndef GDN_STEP_NT
#define GDN_STEP_NT 1024
#endif

template <int DK, bool DB, typename XT, typename CT, typename WT, typename OT>
__global__ __launch_bounds__(GDN_STEP_NT) void decode_step_kernel(
    const XT* __restrict__ x, const GateArgs ga,
    const int32_t* __restrict__ slot, CT* __restrict__ cs, const WT* __restrict__ w,
    const WT* __restrict__ bias, float* __restrict__ rec, OT* __restrict__ out, int32_t H,
    int32_t HV, int32_t dv, int32_t n_groups, float scale, int32_t flags,
    const int32_t* __restrict__ err_flag) {
    constexpr int NV = DK / 32;               // float4 per lane per row
    extern __shared__ float ys[];             // [q_h (DK) | k_h (DK) | v of the group (G dv) | (g, beta) x G]
    if (call_rejected(err_flag)) return;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane & 7;
    constexpr int NT = GDN_STEP_NT;
    constexpr int RP = NT / 8;                // state rows per pass
    const int rl = wave * 8 + (lane >> 3);    // row within a pass
    const int G = HV / H;
    const int R = G * dv;                     // state rows of the group
    const int D = 2 * H * DK + HV * dv;
    const int units = (2 * DK + R) / 4;       // conv work: 4 channels per unit

    for (int grp = blockIdx.x; grp < n_groups; grp += gridDim.x) {
        const int b = grp / H;
        const int h = grp - b * H;
        const int32_t s = slot[b];
        OT* ob = out + (static_cast<size_t>(b) * HV + static_cast<size_t>(h) * G) * dv;
        if (s <= 0) {                         // inactive row: zeros, caches untouched
            for (int r = threadIdx.x; r < R; r += NT) elem<OT>::st(ob + r, 0.0f);
            continue;
        }
        float* Sg = rec + ((static_cast<size_t>(s) * HV + static_cast<size_t>(h) * G) * dv) * DK;

        // Rows past the group (a partial last pass) re-read the group's last
        // row, which the pass then skips: the registers are always defined, so
        // no value has to survive from an earlier group (12-16 fewer VGPRs).
        auto fetch = [&](float4 (&St)[NV], int r0) {
            const int r = min(r0 + rl, R - 1);
#pragma unroll
            for (int i = 0; i < NV; ++i)
                St[i] = state_ld(Sg + static_cast<size_t>(r) * DK + 32 * i + 4 * sub);
        };
        float4 S[NV], S2[NV];

        // conv of the group's channels into LDS (and the in-place roll).  With
        // one 4-channel unit per thread, the unit's loads go out first and the
        // first pass's state loads after them, so the conv math waits for its
        // own loads only and the state rows are in flight during it.
        const XT* xb = x + static_cast<size_t>(b) * D;
        CT* csb = cs + static_cast<size_t>(s) * D * (CONV_W - 1);
        auto channel = [&](int lc) {
            return (lc < DK) ? h * DK + lc
                 : (lc < 2 * DK) ? H * DK + h * DK + (lc - DK)
                                 : 2 * H * DK + h * R + (lc - 2 * DK);
        };
        const bool silu_on = (flags & GDN_FLAG_SILU) != 0;
        float* gs = ys + 2 * DK + R;          // gates of the group's value heads
        float gx0 = 0.0f, gx1 = 0.0f;
        GateHead gh{0.0f, 0.0f};
        const bool gate_lane = static_cast<int>(threadIdx.x) < G;
        if (gate_lane) {                      // issued before the conv and state loads
            gate_raw(ga, static_cast<size_t>(b) * HV + h * G + threadIdx.x, gx0, gx1);
            gh = gate_head(ga, h * G + threadIdx.x);
        }
        if (units <= NT) {
            // threads past the last unit re-read unit 0 (loads stay unconditional)
            const bool mine = static_cast<int>(threadIdx.x) < units;
            const int lc = mine ? 4 * static_cast<int>(threadIdx.x) : 0;
            const int c = channel(lc);
            Conv4In<XT, CT, WT> in;
            conv4_load<XT, CT, WT>(xb + c, csb + static_cast<size_t>(c) * (CONV_W - 1), w + c * CONV_W,
                                   bias ? bias + c : nullptr, in);
            fetch(S, 0);
            if (DB && RP < R) fetch(S2, RP);
            if (mine) {
                float y[4];
                conv4_finish<XT, CT, WT>(in, csb + static_cast<size_t>(c) * (CONV_W - 1), silu_on, y);
                *reinterpret_cast<float4*>(&ys[lc]) = make_float4(y[0], y[1], y[2], y[3]);
            }
        } else {
            for (int u = threadIdx.x; u < units; u += NT) {
                const int lc = 4 * u;
                const int c = channel(lc);
                float y[4];
                conv4_token<XT, CT, WT>(xb + c, csb + static_cast<size_t>(c) * (CONV_W - 1), w + c * CONV_W,
                                        bias ? bias + c : nullptr, silu_on, y);
                *reinterpret_cast<float4*>(&ys[lc]) = make_float4(y[0], y[1], y[2], y[3]);
            }
            fetch(S, 0);
            if (DB && RP < R) fetch(S2, RP);
        }
        if (gate_lane) {
            float gv, bv;
            gate_finish(ga, gh, gx0, gx1, gv, bv);
            gs[2 * threadIdx.x] = gv;
            gs[2 * threadIdx.x + 1] = bv;
        }
        for (int t = threadIdx.x + NT; t < G; t += NT) {     // groups of more than NT heads
            float x0, x1, gv, bv;
            gate_raw(ga, static_cast<size_t>(b) * HV + h * G + t, x0, x1);
            gate_finish(ga, gate_head(ga, h * G + t), x0, x1, gv, bv);
            gs[2 * t] = gv;
            gs[2 * t + 1] = bv;
        }
        __syncthreads();

        float4 qf[NV], kf[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            qf[i] = *reinterpret_cast<const float4*>(&ys[32 * i + 4 * sub]);
            kf[i] = *reinterpret_cast<const float4*>(&ys[DK + 32 * i + 4 * sub]);
        }
        float qmul = scale, kmul = 1.0f;
        if (flags & GDN_FLAG_QK_L2NORM) {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                sq = fmaf(qf[i].x, qf[i].x, sq); sq = fmaf(qf[i].y, qf[i].y, sq);
                sq = fmaf(qf[i].z, qf[i].z, sq); sq = fmaf(qf[i].w, qf[i].w, sq);
                sk = fmaf(kf[i].x, kf[i].x, sk); sk = fmaf(kf[i].y, kf[i].y, sk);
                sk = fmaf(kf[i].z, kf[i].z, sk); sk = fmaf(kf[i].w, kf[i].w, sk);
            }
            sq = sum8(sq);
            sk = sum8(sk);
            qmul = scale / sqrtf(sq + 1e-6f);
            kmul = 1.0f / sqrtf(sk + 1e-6f);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            qf[i].x *= qmul; qf[i].y *= qmul; qf[i].z *= qmul; qf[i].w *= qmul;
            kf[i].x *= kmul; kf[i].y *= kmul; kf[i].z *= kmul; kf[i].w *= kmul;
        }

        // the passes: pass 0's rows are already in S
        auto pass = [&](float4 (&S)[NV], int r0) {
            const int r = r0 + rl;
            if (r >= R) return;               // the 8 lanes of a row share the test
            const int gi = r / dv;            // this row's value head within the group
            const float alpha = expf(gs[2 * gi]);
            const float bt = gs[2 * gi + 1];
            const float vr = ys[2 * DK + r];
            float u = 0.f;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                S[i].x *= alpha; S[i].y *= alpha; S[i].z *= alpha; S[i].w *= alpha;
                u = fmaf(S[i].x, kf[i].x, u); u = fmaf(S[i].y, kf[i].y, u);
                u = fmaf(S[i].z, kf[i].z, u); u = fmaf(S[i].w, kf[i].w, u);
            }
            u = sum8(u);
            const float delta = bt * (vr - u);
            float o = 0.f;
            int qo = 4 * sub;
            if constexpr (DB) asm volatile("" : "+v"(qo));   // no reuse across rows
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                S[i].x = fmaf(delta, kf[i].x, S[i].x); S[i].y = fmaf(delta, kf[i].y, S[i].y);
                S[i].z = fmaf(delta, kf[i].z, S[i].z); S[i].w = fmaf(delta, kf[i].w, S[i].w);
                float4 qv = qf[i];
                if constexpr (DB) {
                    qv = *reinterpret_cast<const float4*>(&ys[32 * i + qo]);
                    qv.x *= qmul; qv.y *= qmul; qv.z *= qmul; qv.w *= qmul;
                }
                o = fmaf(S[i].x, qv.x, o); o = fmaf(S[i].y, qv.y, o);
                o = fmaf(S[i].z, qv.z, o); o = fmaf(S[i].w, qv.w, o);
            }
            o = sum8(o);
#pragma unroll
            for (int i = 0; i < NV; ++i) state_st(Sg + static_cast<size_t>(r) * DK + 32 * i + 4 * sub, S[i]);
            if (sub == 0) elem<OT>::st(ob + r, o);
        };
        if constexpr (DB) {
            for (int r0 = 0; r0 < R; r0 += 2 * RP) {
                pass(S, r0);
                if (r0 + 2 * RP < R) fetch(S, r0 + 2 * RP);
                pass(S2, r0 + RP);
                if (r0 + 3 * RP < R) fetch(S2, r0 + 3 * RP);
            }
        } else {
            pass(S, 0);
            for (int r0 = RP; r0 < R; r0 += RP) {
                fetch(S, r0);
                pass(S, r0);
            }
        }
        __syncthreads();                      // ys is rewritten by the next group
    }
}

// Compute units of the current device, asked of the runtime on every call
// (no cache is kept).
int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

namespace {
struct RecArgs {
    const void* y; GateArgs gate; const int32_t* slot; int32_t batch;
    float* rec; void* out; const gdn_dims* d; float scale; int32_t flags; const int32_t* err;
    hipStream_t st;
};



template <int DK, int RPL, bool FULL, bool GATED, typename YT, typename OT>
hipError_t run_rec_g(const RecArgs& a) {
    const int rows_per_wg = 32 * RPL;
    const int tiles = (a.d->head_v_dim + rows_per_wg - 1) / rows_per_wg;
    const int64_t items = static_cast<int64_t>(a.batch) * a.d->num_v_heads * tiles;
    const int64_t resident = static_cast<int64_t>(cu_count()) * GDN_DECODE_WG_PER_CU;
    const int grid = static_cast<int>(items < resident ? items : resident);
    return launch(decode_rec_kernel<DK, RPL, FULL, GATED, YT, OT>, dim3(grid), dim3(256), 0, a.st,
                  static_cast<const YT*>(a.y), a.gate, a.slot, a.rec,
                  static_cast<OT*>(a.out), a.d->num_k_heads, a.d->num_v_heads,
                  a.d->head_v_dim, tiles, static_cast<int32_t>(items), a.scale, a.flags, a.err);
}

template <int DK, int RPL, bool FULL, typename YT, typename OT>
hipError_t run_rec_t(const RecArgs& a) {
    if (a.gate.a) return run_rec_g<DK, RPL, FULL, true, YT, OT>(a);
    return run_rec_g<DK, RPL, FULL, false, YT, OT>(a);
}

template <int DK, int RPL, typename YT, typename OT>
hipError_t run_rec(const RecArgs& a) {
    if (a.d->head_v_dim % (32 * RPL) == 0) return run_rec_t<DK, RPL, true, YT, OT>(a);
    return run_rec_t<DK, RPL, false, YT, OT>(a);
}

// Rows per lane: as many 32-row steps as the head needs (up to 4), so one
// workgroup streams a whole head of up to 128 rows; the per-row arithmetic is
// identical for every choice.
template <int DK, typename YT, typename OT>
hipError_t pick_rpl(const RecArgs& a) {
    const int dv = a.d->head_v_dim;
    if (dv > 64 && GDN_DECODE_RPL_MAX >= 4) return run_rec<DK, 4, YT, OT>(a);
    if (dv > 32 && GDN_DECODE_RPL_MAX >= 2) return run_rec<DK, 2, YT, OT>(a);
    return run_rec<DK, 1, YT, OT>(a);
}

template <typename YT, typename OT>
hipError_t pick_dk(const RecArgs& a) {
    switch (a.d->head_k_dim) {
        case 32: return pick_rpl<32, YT, OT>(a);
        case 64: return pick_rpl<64, YT, OT>(a);
        case 128: return pick_rpl<128, YT, OT>(a);
        case 256: return pick_rpl<256, YT, OT>(a);
        default: return hipErrorInvalidValue;
    }
}
}  // namespace

// Workgroups per CU in the fused step's grid (a group-strided loop beyond it).
// Measured at batch 256: one workgroup per group (4096) 206 us; one or two
// resident per CU looping over groups 211 us; at batch 1024 (16384 groups) a
// 4096 grid looping over four groups each 823 us, one per group 793 us.
#ifndef GDN_STEP_WG_PER_CU
#define GDN_STEP_WG_PER_CU 256
#endif
// Double-buffered passes up to this many groups per CU (see decode_step_kernel).
// Measured: batch 32 (2 groups per CU) 30.1 us vs 30.5 single-buffered; batch
// 64 56.7 vs 55.7; batch 256 206.7 vs 203.6.
#ifndef GDN_STEP_DB_MAX_GROUPS_PER_CU
#define GDN_STEP_DB_MAX_GROUPS_PER_CU 2
#endif

namespace {
struct StepArgs {
    const void* x; GateArgs gate; const int32_t* slot; int32_t batch;
    void* cs; const void* w; const void* bias; float* rec; void* out; const gdn_dims* d;
    float scale; int32_t flags; const int32_t* err; hipStream_t st;
};

template <int DK, typename XT, typename CT, typename WT, typename OT>
hipError_t run_step(const StepArgs& a) {
    const int G = a.d->num_v_heads / a.d->num_k_heads;
    const size_t lds = static_cast<size_t>(2 * DK + G * a.d->head_v_dim + 2 * G) * sizeof(float);
    const int64_t groups = static_cast<int64_t>(a.batch) * a.d->num_k_heads;
    const int64_t resident = static_cast<int64_t>(cu_count()) * GDN_STEP_WG_PER_CU;
    const int grid = static_cast<int>(groups < resident ? groups : resident);
    // dk > 128 keeps single buffering: its 32 state registers per pass would
    // not fit twice
    const bool db = DK <= 128 &&
                    groups <= static_cast<int64_t>(cu_count()) * GDN_STEP_DB_MAX_GROUPS_PER_CU;
    auto kern = db ? decode_step_kernel<DK, (DK <= 128), XT, CT, WT, OT>
                   : decode_step_kernel<DK, false, XT, CT, WT, OT>;
    return launch(kern, dim3(grid), dim3(GDN_STEP_NT), lds, a.st,
                  static_cast<const XT*>(a.x), a.gate, a.slot, static_cast<CT*>(a.cs),
                  static_cast<const WT*>(a.w), static_cast<const WT*>(a.bias), a.rec,
                  static_cast<OT*>(a.out), a.d->num_k_heads, a.d->num_v_heads,
                  a.d->head_v_dim, static_cast<int32_t>(groups), a.scale, a.flags, a.err);
}

template <int DK, typename XT, typename CT, typename WT>
hipError_t step_o(gdn_dtype o, const StepArgs& a) {
    return o == GDN_BF16 ? run_step<DK, XT, CT, WT, bf16_t>(a) : run_step<DK, XT, CT, WT, float>(a);
}
template <int DK, typename XT, typename CT>
hipError_t step_w(gdn_dtype wt, gdn_dtype o, const StepArgs& a) {
    return wt == GDN_BF16 ? step_o<DK, XT, CT, bf16_t>(o, a) : step_o<DK, XT, CT, float>(o, a);
}
template <int DK, typename XT>
hipError_t step_c(gdn_dtype c, gdn_dtype wt, gdn_dtype o, const StepArgs& a) {
    return c == GDN_BF16 ? step_w<DK, XT, bf16_t>(wt, o, a) : step_w<DK, XT, float>(wt, o, a);
}
template <int DK>
hipError_t step_x(gdn_dtype xt, gdn_dtype c, gdn_dtype wt, gdn_dtype o, const StepArgs& a) {
    return xt == GDN_BF16 ? step_c<DK, bf16_t>(c, wt, o, a) : step_c<DK, float>(c, wt, o, a);
}
}  // namespace

// The fused step is chosen while each (row, key head) group has at most
// GDN_DECODE_FUSED_MAX_CUS_PER_GROUP CUs to itself and there are at most
// GDN_DECODE_FUSED_MAX_GROUPS_PER_CU groups per CU.  Measured (graph replay per
// step, H = 16, HV = 32, d = 128, 256 CUs, 1024-thread groups, the recurrence
// kernel with one workgroup per item), fused vs the conv + recurrence pair:
// batch 1024 811.4 vs 797.6 us; 256 204.8 vs 193.1; 128 103.7 vs 97.8; 64 56.2
// vs 54.0; 32 30.1 vs 29.7; 16 14.5 vs 17.2; 8 11.1 vs 11.3; 4 7.8 vs 7.7.
// With one or two groups per CU the fused kernel's double-buffered passes hide
// its latency chain; past that, the pair's small recurrence items (no barrier,
// several workgroups per CU) stream the state faster than one 1024-thread
// group per CU, the conv kernel and the activations' round trip included.
// Below a quarter group per CU the pair's items also spread the few rows over
// more CUs (batch 2: 8.7 vs 7.4 us, batch 1: 8.5 vs 7.0).
#ifndef GDN_DECODE_FUSED_MAX_CUS_PER_GROUP
#define GDN_DECODE_FUSED_MAX_CUS_PER_GROUP 4
#endif
#ifndef GDN_DECODE_FUSED_MAX_GROUPS_PER_CU
#define GDN_DECODE_FUSED_MAX_GROUPS_PER_CU 1
#endif

bool decode_step_fused_fits(const gdn_dims& d) {
    const int64_t G = d.num_v_heads / d.num_k_heads;
    const int64_t lds = (2LL * d.head_k_dim + G * d.head_v_dim + 2 * G) * static_cast<int64_t>(sizeof(float));
    return lds <= 65536;
}

bool decode_step_use_fused(const gdn_dims& d, int32_t batch) {
    // dk > 128 stays on the pair: the 1024-thread fused kernel (128 VGPRs)
    // spills its per-row registers there
    const int64_t groups = static_cast<int64_t>(batch) * d.num_k_heads;
    const int64_t cus = cu_count();
    return decode_step_fused_fits(d) && d.head_k_dim <= 128 &&
           groups * GDN_DECODE_FUSED_MAX_CUS_PER_GROUP >= cus &&
           groups <= cus * GDN_DECODE_FUSED_MAX_GROUPS_PER_CU;
}

hipError_t launch_decode_step_fused(const void* x, gdn_dtype x_dt, const GateArgs& gate,
                                    const int32_t* slot_idx, int32_t batch,
                                    void* conv_state, gdn_dtype cs_dt, const void* weight,
                                    const void* bias, gdn_dtype w_dt, float* rec_state, void* out,
                                    gdn_dtype out_dt, const gdn_dims& dims, float scale,
                                    int32_t flags, const int32_t* err_flag, hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    const StepArgs a{x, gate, slot_idx, batch, conv_state, weight, bias, rec_state, out,
                     &dims, scale, flags, err_flag, stream};
    switch (dims.head_k_dim) {
        case 32: return step_x<32>(x_dt, cs_dt, w_dt, out_dt, a);
        case 64: return step_x<64>(x_dt, cs_dt, w_dt, out_dt, a);
        case 128: return step_x<128>(x_dt, cs_dt, w_dt, out_dt, a);
        case 256: return step_x<256>(x_dt, cs_dt, w_dt, out_dt, a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_rec(const void* y, gdn_dtype y_dt, const GateArgs& gate,
                             const int32_t* slot_idx, int32_t batch, float* rec_state,
                             void* out, gdn_dtype out_dt, const gdn_dims& dims, float scale,
                             int32_t flags, const int32_t* err_flag, hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    const RecArgs a{y, gate, slot_idx, batch, rec_state, out, &dims, scale, flags, err_flag,
                    stream};
    if (y_dt == GDN_BF16)
        return out_dt == GDN_BF16 ? pick_dk<bf16_t, bf16_t>(a) : pick_dk<bf16_t, float>(a);
    return out_dt == GDN_BF16 ? pick_dk<float, bf16_t>(a) : pick_dk<float, float>(a);
}

}  // namespace gdn
