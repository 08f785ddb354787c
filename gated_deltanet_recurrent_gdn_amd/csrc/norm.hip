// norm.hip -- gated RMSNorm of the GDN block's output.
//
// RL-Kernel PR #469, "Latest Status": the block's output goes through a gated
// RMSNorm (SiLU or sigmoid gate, optional zero-centred weight, i.e. weight + 1).
// The pages print no formula; the plain definition is used, norm before gate:
//   out[r, j] = x[r, j] / sqrt(sum_j x[r, j]^2 / dim + eps) * w'[j] * act(z[r, j]).
//
// A row takes L lanes, L the power of two that covers dim / 4 (at most 64),
// so a wave holds 64 / L rows (two rows of 128 per wave); each lane keeps its
// groups of 4 elements in registers, so out may alias x.  The sum of squares
// is an in-lane fma chain followed by a fixed butterfly over the row's L lanes
// (DPP inside 16-lane rows, then the xor-16 and xor-32 exchanges) whose every
// step adds a symmetric pair, so the row's lanes hold the bitwise-same total
// and the result never depends on the batch.  HBM-bound: x and z read once,
// out written once.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {

// G consecutive elements (4 or 8) as fp32: one 8- or 16-byte access for bf16,
// one or two 16-byte accesses for fp32.
template <typename T, int G> struct VecG;
template <int G> struct VecG<float, G> {
    __device__ __forceinline__ static void ld(const float* p, float (&v)[G]) {
#pragma unroll
        for (int h = 0; h < G / 4; ++h) {
            const float4 f = *reinterpret_cast<const float4*>(p + 4 * h);
            v[4 * h] = f.x; v[4 * h + 1] = f.y; v[4 * h + 2] = f.z; v[4 * h + 3] = f.w;
        }
    }
    __device__ __forceinline__ static void st(float* p, const float (&v)[G]) {
#pragma unroll
        for (int h = 0; h < G / 4; ++h)
            *reinterpret_cast<float4*>(p + 4 * h) = make_float4(v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]);
    }
};
template <> struct VecG<bf16_t, 4> {
    __device__ __forceinline__ static void ld(const bf16_t* p, float (&v)[4]) {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        v[0] = bf16lo_to_f32(u.x); v[1] = bf16hi_to_f32(u.x); v[2] = bf16lo_to_f32(u.y); v[3] = bf16hi_to_f32(u.y);
    }
    __device__ __forceinline__ static void st(bf16_t* p, const float (&v)[4]) {
        *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
};
template <> struct VecG<bf16_t, 8> {
    __device__ __forceinline__ static void ld(const bf16_t* p, float (&v)[8]) {
        const uint4 u = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) { v[2 * j] = bf16lo_to_f32(w[j]); v[2 * j + 1] = bf16hi_to_f32(w[j]); }
    }
    __device__ __forceinline__ static void st(bf16_t* p, const float (&v)[8]) {
        *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
};

// Sum over aligned groups of L lanes (L a power of two, uniform).
__device__ __forceinline__ float group_sum_sym(float x, int L) {
    if (L >= 2) x = x + dpp<DPP_QUAD_XOR1>(x);
    if (L >= 4) x = x + dpp<DPP_QUAD_XOR2>(x);
    if (L >= 8) x = x + dpp<DPP_HALF_MIRROR>(x);
    if (L >= 16) x = x + dpp<DPP_ROW_MIRROR>(x);   // lanes i and 15 - i: the two 8-lane halves
    if (L >= 32) x = x + __shfl_xor(x, 16, 64);
    if (L >= 64) x = x + __shfl_xor(x, 32, 64);
    return x;
}

template <typename XT, typename WT, typename OT, int G>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(
    const XT* __restrict__ x, const XT* __restrict__ z, const WT* __restrict__ w,
    OT* out, int64_t rows, int32_t dim, int32_t L, float eps, int32_t flags) {
    constexpr int NP = 16 / G;                 // element groups per lane: dim <= 64 * 16
    const int lane = threadIdx.x & 63;
    const int sub = lane & (L - 1);
    const int64_t r = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * (64 / L) + lane / L;
    const bool live = r < rows;            // dead lanes still join the (uniform) butterfly
    const XT* xr = x + (live ? r : 0) * dim;
    float v[NP][G];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int c = G * sub + G * L * i;
#pragma unroll
        for (int e = 0; e < G; ++e) v[i][e] = 0.0f;
        if (live && c < dim) {
            VecG<XT, G>::ld(xr + c, v[i]);
#pragma unroll
            for (int e = 0; e < G; ++e) ss = fmaf(v[i][e], v[i][e], ss);
        }
    }
    ss = group_sum_sym(ss, L);
    if (!live) return;
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(dim) + eps);
    const bool offset = (flags & GDN_NORM_ZERO_CENTRED) != 0;
    const bool sigm = (flags & GDN_NORM_GATE_SIGMOID) != 0;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int c = G * sub + G * L * i;
        if (c >= dim) continue;
        float wv[G], y[G];
        VecG<WT, G>::ld(w + c, wv);
#pragma unroll
        for (int e = 0; e < G; ++e) y[e] = v[i][e] * inv * (offset ? wv[e] + 1.0f : wv[e]);
        if (z) {
            float zv[G];
            VecG<XT, G>::ld(z + r * dim + c, zv);
#pragma unroll
            for (int e = 0; e < G; ++e) {
                // sigmoid by the hardware reciprocal (1 ulp) of 1 + e^-z
                const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-zv[e]));
                y[e] *= sigm ? sg : zv[e] * sg;
            }
        }
        VecG<OT, G>::st(out + r * dim + c, y);
    }
}

template <typename XT, typename WT, typename OT>
hipError_t run_norm(const void* x, const void* z, const void* w, void* out, int64_t rows,
                    int32_t dim, float eps, int32_t flags, hipStream_t st) {
    const int G = (dim % 8 == 0) ? 8 : 4;        // elements per lane group
    int L = 1;
    while (L < 64 && G * L < dim) L *= 2;       // lanes per row
    const int64_t rows_per_block = 4 * (64 / L);
    const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    if (G == 8)
        return launch(gated_rmsnorm_kernel<XT, WT, OT, 8>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                      st, static_cast<const XT*>(x), static_cast<const XT*>(z),
                      static_cast<const WT*>(w), static_cast<OT*>(out), rows, dim, L, eps, flags);
    return launch(gated_rmsnorm_kernel<XT, WT, OT, 4>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st,
                  static_cast<const XT*>(x), static_cast<const XT*>(z), static_cast<const WT*>(w),
                  static_cast<OT*>(out), rows, dim, L, eps, flags);
}

template <typename XT, typename WT>
hipError_t norm_o(gdn_dtype o, const void* x, const void* z, const void* w, void* out, int64_t rows,
                  int32_t dim, float eps, int32_t flags, hipStream_t st) {
    return o == GDN_BF16 ? run_norm<XT, WT, bf16_t>(x, z, w, out, rows, dim, eps, flags, st)
                         : run_norm<XT, WT, float>(x, z, w, out, rows, dim, eps, flags, st);
}
template <typename XT>
hipError_t norm_w(gdn_dtype wt, gdn_dtype o, const void* x, const void* z, const void* w, void* out,
                  int64_t rows, int32_t dim, float eps, int32_t flags, hipStream_t st) {
    return wt == GDN_BF16 ? norm_o<XT, bf16_t>(o, x, z, w, out, rows, dim, eps, flags, st)
                          : norm_o<XT, float>(o, x, z, w, out, rows, dim, eps, flags, st);
}

}  // namespace

hipError_t launch_gated_rmsnorm(const void* x, gdn_dtype x_dt, const void* z, const void* w,
                                gdn_dtype w_dt, void* out, gdn_dtype out_dt, int64_t rows,
                                int32_t dim, float eps, int32_t flags, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    return x_dt == GDN_BF16 ? norm_w<bf16_t>(w_dt, out_dt, x, z, w, out, rows, dim, eps, flags, st)
                            : norm_w<float>(w_dt, out_dt, x, z, w, out, rows, dim, eps, flags, st);
}

}  // namespace gdn
